// Device-side building blocks for gfx950: register-resident block decoders for
// the five weight formats, and the wave-level reductions of the GEMV kernels.
//
// Every decoder works on one 16-byte "chunk" of a weight row (one 128-bit load per
// lane) plus the chunk's scale side data, and offers:
//   * dot<ACT>(chunk, side, xop, acc): acc + (decoded chunk) . (activation slice)
//   * to_f32(chunk, side, out): the exact weights rounded once to fp32 (dequant)
//   * load_x<ACT>(...): the activation slice in the register order dot() consumes,
//     also as fetch_x (the loads only) and prep_x (the conversion), so a kernel can
//     put its weight loads between the two.
// Weights are expanded to bf16 pairs (exact for every format here: at most 8
// significant bits before the block scale) and multiplied with v_dot2_f32_bf16;
// the per-block scale is applied once per block to the fp32 partial sum.
// bf16 activations are used as they are; fp32 activations (the intermediate h)
// are split into hi + lo bf16 parts (16 significant bits) and dotted twice.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq {

enum {
  FMT_MXFP4 = 1,
  FMT_NVFP4 = 2,
  FMT_Q2_K = 3,
  FMT_IQ2_XXS = 4,
  FMT_FP8_B128 = 5,
  FMT_MXFP8 = 6,
  FMT_FP8_B32 = 7,
  FMT_MXFP8_TILED = 8
};
enum { ACT_BF16 = 0, ACT_F32 = 1 };

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Scalar bit casts. Always cast through these: applied directly to an element of
// an ext_vector_type value, __builtin_bit_cast reads the vector's first element.
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, x), acc,
                                         false);
}

// e8m0 code -> 2^(E-127) as fp32 (E = 0 is the subnormal 2^-127, E = 255 is NaN).
__device__ __forceinline__ float e8m0_f32(uint32_t E) {
  uint32_t b = E << 23;
  b = (E == 0u) ? 0x00400000u : b;
  b = (E == 255u) ? 0x7FC00000u : b;
  return __builtin_bit_cast(float, b);
}

__device__ __forceinline__ float half_bits_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Split two fp32 values into hi and lo bf16 pairs with a + b ~ value to 16 bits.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  uint32_t ha = __builtin_bit_cast(uint32_t, a) & 0xFFFF0000u;
  uint32_t hb = __builtin_bit_cast(uint32_t, b) & 0xFFFF0000u;
  float ra = a - __builtin_bit_cast(float, ha);
  float rb = b - __builtin_bit_cast(float, hb);
  hi = (ha >> 16) | hb;
  lo = f32_bf16_rne(ra) | (f32_bf16_rne(rb) << 16);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// -------------------------------------------------------------------------
// Activation slices. XR<ACT>(n) = registers for n weights.
// Every slice is read in two steps so that kernels can issue the loads early and
// convert later: fetch<N> (the 16-byte loads, RawN<ACT, N>::V of them) and
// from_raw<N> (register order for dot()); load<N> does both.
template <int ACT, int N> struct RawN {
  static constexpr int V = (ACT == ACT_BF16) ? N / 8 : N / 4;
};
template <int ACT> struct Act;
template <> struct Act<ACT_BF16> {
  static constexpr int PER_PAIR = 1;
  // n contiguous bf16 values starting at element k0 of row p (n multiple of 8)
  template <int N>
  __device__ static void fetch(const void* row, int k0, u32x4* v) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(row) + k0;
#pragma unroll
    for (int i = 0; i < N / 8; i++) v[i] = ld16(p + 8 * i);
  }
  template <int N>
  __device__ static void from_raw(const u32x4* v, uint32_t* r) {
#pragma unroll
    for (int i = 0; i < N / 8; i++) {
      r[4 * i + 0] = v[i][0];
      r[4 * i + 1] = v[i][1];
      r[4 * i + 2] = v[i][2];
      r[4 * i + 3] = v[i][3];
    }
  }
  template <int N>
  __device__ static void load(const void* row, int k0, uint32_t* r) {
    u32x4 v[N / 8];
    fetch<N>(row, k0, v);
    from_raw<N>(v, r);
  }
  __device__ static float val(const void* row, int k) {
    uint32_t b = reinterpret_cast<const uint16_t*>(row)[k];
    return __builtin_bit_cast(float, b << 16);
  }
};
template <> struct Act<ACT_F32> {
  static constexpr int PER_PAIR = 2;
  // n contiguous fp32 values -> n/2 hi pairs then n/2 lo pairs
  template <int N>
  __device__ static void fetch(const void* row, int k0, u32x4* v) {
    const float* p = reinterpret_cast<const float*>(row) + k0;
#pragma unroll
    for (int i = 0; i < N / 4; i++) v[i] = ld16(p + 4 * i);
  }
  template <int N>
  __device__ static void from_raw(const u32x4* v, uint32_t* r) {
#pragma unroll
    for (int i = 0; i < N / 4; i++) {
      split_pair(u2f(v[i][0]), u2f(v[i][1]), r[2 * i], r[N / 2 + 2 * i]);
      split_pair(u2f(v[i][2]), u2f(v[i][3]), r[2 * i + 1], r[N / 2 + 2 * i + 1]);
    }
  }
  template <int N>
  __device__ static void load(const void* row, int k0, uint32_t* r) {
    u32x4 v[N / 4];
    fetch<N>(row, k0, v);
    from_raw<N>(v, r);
  }
  __device__ static float val(const void* row, int k) { return reinterpret_cast<const float*>(row)[k]; }
};

// dot of a bf16 weight pair with activation pair j of a slice of N weights
template <int ACT, int N>
__device__ __forceinline__ float dotp(uint32_t w, const uint32_t* x, int j, float acc) {
  acc = dot2(w, x[j], acc);
  if (ACT != ACT_BF16) acc = dot2(w, x[N / 2 + j], acc);
  return acc;
}

// -------------------------------------------------------------------------
// Weight tensor view for one expert.
struct WView {
  const uint8_t* data;    // expert's data plane
  const uint8_t* scales;  // expert's scale plane
  int rows, cols;
};

// The IQ2_XXS GEMV takes its sign words from the LDS table (1) or makes them in
// registers (0); the token-grouped kernels always use the table.
#ifndef MOEQ_IQ2_SIGN_LDS
#define MOEQ_IQ2_SIGN_LDS 0
#endif
struct Iq2Lds {
  uint32_t grid[256 * 4];  // codebook entry i as four bf16 pairs (values 0..255: sign bits clear)
  u32x4 sgn[128];          // the four bf16-pair sign words of 7-bit sign code c (iq2_sign_words)
};

template <int FMT> struct Dec;

// MXFP4: chunk = 16 nibble bytes = one 32-weight block; side = its e8m0 code.
template <> struct Dec<FMT_MXFP4> {
  static constexpr int WPC = 32;
  typedef uint32_t Side;
  __device__ static Side side(const WView& w, int r, int ch) { return w.scales[(size_t)r * (w.cols / 32) + ch]; }
  __device__ static const uint8_t* chunk_ptr(const WView& w, int r, int ch) {
    return w.data + (size_t)r * (w.cols / 2) + (size_t)ch * 16;
  }
  template <int ACT>
  __device__ static int xregs() { return 16 * Act<ACT>::PER_PAIR; }
  template <int ACT>
  __device__ static void fetch_x(const void* row, int ch, u32x4* raw) {
    Act<ACT>::template fetch<32>(row, ch * 32, raw);
  }
  template <int ACT>
  __device__ static void prep_x(const u32x4* raw, uint32_t* x, float*) {
    Act<ACT>::template from_raw<32>(raw, x);
  }
  template <int ACT>
  __device__ static void load_x(const void* row, int ch, uint32_t* x, float*) {
    Act<ACT>::template load<32>(row, ch * 32, x);
  }
  template <int ACT>
  __device__ static float dot(u32x4 q, Side s, const uint32_t* x, const float* /*xs*/, float acc, const Iq2Lds*) {
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      p = dotp<ACT, 32>(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], 1.0f, 0)), x,
                        4 * i + 0, p);
      p = dotp<ACT, 32>(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], 1.0f, 1)), x,
                        4 * i + 1, p);
      p = dotp<ACT, 32>(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], 1.0f, 2)), x,
                        4 * i + 2, p);
      p = dotp<ACT, 32>(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], 1.0f, 3)), x,
                        4 * i + 3, p);
    }
    return __builtin_fmaf(p, e8m0_f32(s), acc);
  }
  // out[j] = weight at column ch*32 + j
  __device__ static void to_f32(u32x4 q, Side s, float scale2, const uint8_t*, float* out) {
    (void)scale2;
    int ex = (int)s - 127;
#pragma unroll
    for (int i = 0; i < 4; i++) {
#define MOEQ_FP4F(B)                                                        \
  {                                                                         \
    f32x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[i], 1.0f, B);   \
    out[8 * i + 2 * B] = __builtin_ldexpf(v.x, ex);                         \
    out[8 * i + 2 * B + 1] = __builtin_ldexpf(v.y, ex);                     \
  }
      MOEQ_FP4F(0) MOEQ_FP4F(1) MOEQ_FP4F(2) MOEQ_FP4F(3)
#undef MOEQ_FP4F
    }
    if (s == 255u) {
#pragma unroll
      for (int j = 0; j < 32; j++) out[j] = __builtin_nanf("");
    }
  }
  __device__ static int out_col(int ch, int j) { return ch * 32 + j; }
};

// NVFP4: chunk = 16 nibble bytes = two 16-weight blocks; side = their two e4m3 codes.
template <> struct Dec<FMT_NVFP4> {
  static constexpr int WPC = 32;
  typedef uint32_t Side;
  __device__ static Side side(const WView& w, int r, int ch) {
    return *reinterpret_cast<const uint16_t*>(w.scales + (size_t)r * (w.cols / 16) + 2 * ch);
  }
  __device__ static const uint8_t* chunk_ptr(const WView& w, int r, int ch) {
    return w.data + (size_t)r * (w.cols / 2) + (size_t)ch * 16;
  }
  template <int ACT>
  __device__ static void fetch_x(const void* row, int ch, u32x4* raw) {
    Act<ACT>::template fetch<32>(row, ch * 32, raw);
  }
  template <int ACT>
  __device__ static void prep_x(const u32x4* raw, uint32_t* x, float*) {
    Act<ACT>::template from_raw<32>(raw, x);
  }
  template <int ACT>
  __device__ static void load_x(const void* row, int ch, uint32_t* x, float*) {
    Act<ACT>::template load<32>(row, ch * 32, x);
  }
  template <int ACT>
  __device__ static float dot(u32x4 q, Side s, const uint32_t* x, const float*, float acc, const Iq2Lds*) {
    f32x2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s, 1.0f, false);
#pragma unroll
    for (int b = 0; b < 2; b++) {
      float p = 0.f;
#pragma unroll
      for (int i = 2 * b; i < 2 * b + 2; i++) {
        p = dotp<ACT, 32>(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], 1.0f, 0)), x,
                          4 * i + 0, p);
        p = dotp<ACT, 32>(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], 1.0f, 1)), x,
                          4 * i + 1, p);
        p = dotp<ACT, 32>(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], 1.0f, 2)), x,
                          4 * i + 2, p);
        p = dotp<ACT, 32>(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], 1.0f, 3)), x,
                          4 * i + 3, p);
      }
      acc = __builtin_fmaf(p, b == 0 ? sc.x : sc.y, acc);
    }
    return acc;
  }
  __device__ static void to_f32(u32x4 q, Side s, float scale2, const uint8_t*, float* out) {
    f32x2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s, 1.0f, false);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float e = i < 2 ? sc.x : sc.y;
#define MOEQ_FP4N(B)                                                       \
  {                                                                        \
    f32x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[i], 1.0f, B);  \
    out[8 * i + 2 * B] = (v.x * e) * scale2;                               \
    out[8 * i + 2 * B + 1] = (v.y * e) * scale2;                           \
  }
      MOEQ_FP4N(0) MOEQ_FP4N(1) MOEQ_FP4N(2) MOEQ_FP4N(3)
#undef MOEQ_FP4N
    }
  }
  __device__ static int out_col(int ch, int j) { return ch * 32 + j; }
};

// Q2_K: chunk = quarter c of a superblock's 64 qs bytes; it holds the 2-bit quants
// of four 16-weight sub-blocks (one per crumb position p), weights
// 128h + 32p + 16(c&1) + i, i < 16, with h = c >> 1. Crumbs are expanded with a
// magic bias: OR-ing a crumb into the mantissa of bf16 1.0 gives 1 + q * 2^-f, so
// sum((1 + q 2^-f) x) = sum(x) + 2^-f sum(q x); the per-sub-block sum of x is
// precomputed with the activation slice and removed with the min term:
//   contribution = A * S - (A + dmin * m) * sum(x),  A = d * sc * 2^f.
template <> struct Dec<FMT_Q2_K> {
  static constexpr int WPC = 64;
  struct Side {
    uint32_t lo, hi;  // the 8 scale bytes of this half (bytes (c&1) + 2p are ours)
    uint32_t dd;      // d | dmin << 16
  };
  __device__ static Side side(const WView& w, int r, int ch) {
    int sb = ch >> 2, c = ch & 3;
    const uint8_t* p = w.scales + ((size_t)r * (w.cols / 256) + sb) * 20;
    const uint32_t* p32 = reinterpret_cast<const uint32_t*>(p);
    Side s;
    s.lo = p32[2 * (c >> 1)] >> (8 * (c & 1));
    s.hi = p32[2 * (c >> 1) + 1] >> (8 * (c & 1));
    s.dd = *reinterpret_cast<const uint32_t*>(p + 16);
    return s;
  }
  __device__ static const uint8_t* chunk_ptr(const WView& w, int r, int ch) {
    return w.data + (size_t)r * (w.cols / 256) * 64 + (size_t)ch * 16;
  }
  __device__ static int seg_base(int ch, int p) {
    int sb = ch >> 2, c = ch & 3;
    return sb * 256 + 128 * (c >> 1) + 32 * p + 16 * (c & 1);
  }
  // x layout: for p < 4, i < 4: pair A (bytes 0,2 of word i) at 8p + 2i, pair B
  // (bytes 1,3) at 8p + 2i + 1. xs[p] = sum of the 16 activations of sub-block p.
  template <int ACT>
  __device__ static void fetch_x(const void* row, int ch, u32x4* raw) {
    constexpr int R = RawN<ACT, 16>::V;
#pragma unroll
    for (int p = 0; p < 4; p++) Act<ACT>::template fetch<16>(row, seg_base(ch, p), raw + R * p);
  }
  template <int ACT>
  __device__ static void prep_x(const u32x4* raw, uint32_t* x, float* xs) {
    constexpr int R = RawN<ACT, 16>::V;
#pragma unroll
    for (int p = 0; p < 4; p++) {
      const u32x4* v = raw + R * p;
      float s = 0.f;
      if (ACT == ACT_BF16) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          uint32_t w0 = v[i >> 1][2 * (i & 1)], w1 = v[i >> 1][2 * (i & 1) + 1];  // (x0,x1), (x2,x3)
          x[8 * p + 2 * i] = (w0 & 0xFFFFu) | (w1 << 16);                           // (x0, x2)
          x[8 * p + 2 * i + 1] = (w0 >> 16) | (w1 & 0xFFFF0000u);                   // (x1, x3)
          s += __builtin_bit_cast(float, w0 << 16) + __builtin_bit_cast(float, w0 & 0xFFFF0000u) +
               __builtin_bit_cast(float, w1 << 16) + __builtin_bit_cast(float, w1 & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          uint32_t h02, l02, h13, l13;
          split_pair(u2f(v[i][0]), u2f(v[i][2]), h02, l02);
          split_pair(u2f(v[i][1]), u2f(v[i][3]), h13, l13);
          x[8 * p + 2 * i] = h02;
          x[32 + 8 * p + 2 * i] = l02;
          x[8 * p + 2 * i + 1] = h13;
          x[32 + 8 * p + 2 * i + 1] = l13;
          // The bias term removed below must be the sum of exactly the values the
          // dot products see (hi + lo), or the split's residual would not cancel.
          s += (u2f(h02 << 16) + u2f(l02 << 16)) + (u2f(h13 << 16) + u2f(l13 << 16)) +
               (u2f(h02 & 0xFFFF0000u) + u2f(l02 & 0xFFFF0000u)) + (u2f(h13 & 0xFFFF0000u) + u2f(l13 & 0xFFFF0000u));
        }
      }
      xs[p] = s;
    }
  }
  template <int ACT>
  __device__ static void load_x(const void* row, int ch, uint32_t* x, float* xs) {
    u32x4 raw[4 * RawN<ACT, 16>::V];
    fetch_x<ACT>(row, ch, raw);
    prep_x<ACT>(raw, x, xs);
  }
  template <int ACT>
  __device__ static float dot(u32x4 q, Side s, const uint32_t* x, const float* xs, float acc, const Iq2Lds*) {
    const uint32_t ONE = 0x3F803F80u;
    float S[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      uint32_t w = q[i], w8 = q[i] >> 8;
      uint32_t a0 = (w & 0x00030003u) | ONE, b0 = (w8 & 0x00030003u) | ONE;       // 1 + q/128
      uint32_t a1 = (w & 0x000C000Cu) | ONE, b1 = (w8 & 0x000C000Cu) | ONE;       // 1 + q/32
      uint32_t a2 = (w & 0x00300030u) | ONE, b2 = (w8 & 0x00300030u) | ONE;       // 1 + q/8
      uint32_t a3 = ((w >> 1) & 0x00600060u) | ONE, b3 = ((w8 >> 1) & 0x00600060u) | ONE;  // 1 + q/4
      S[0] = dotp<ACT, 64>(a0, x, 0 + 2 * i, S[0]);
      S[0] = dotp<ACT, 64>(b0, x, 0 + 2 * i + 1, S[0]);
      S[1] = dotp<ACT, 64>(a1, x, 8 + 2 * i, S[1]);
      S[1] = dotp<ACT, 64>(b1, x, 8 + 2 * i + 1, S[1]);
      S[2] = dotp<ACT, 64>(a2, x, 16 + 2 * i, S[2]);
      S[2] = dotp<ACT, 64>(b2, x, 16 + 2 * i + 1, S[2]);
      S[3] = dotp<ACT, 64>(a3, x, 24 + 2 * i, S[3]);
      S[3] = dotp<ACT, 64>(b3, x, 24 + 2 * i + 1, S[3]);
    }
    float d = half_bits_f32(s.dd), dmin = half_bits_f32(s.dd >> 16);
    const float F[4] = {128.f, 32.f, 8.f, 4.f};
#pragma unroll
    for (int p = 0; p < 4; p++) {
      uint32_t byte = ((p < 2 ? s.lo : s.hi) >> (16 * (p & 1))) & 0xFFu;
      float A = d * F[p] * (float)(byte & 15u);
      float B = __builtin_fmaf(dmin, (float)(byte >> 4), A);
      acc = __builtin_fmaf(A, S[p], acc);
      acc = __builtin_fmaf(-B, xs[p], acc);
    }
    return acc;
  }
  __device__ static void to_f32(u32x4 q, Side s, float, const uint8_t*, float* out) {
    float d = half_bits_f32(s.dd), dmin = half_bits_f32(s.dd >> 16);
#pragma unroll
    for (int p = 0; p < 4; p++) {
      uint32_t byte = ((p < 2 ? s.lo : s.hi) >> (16 * (p & 1))) & 0xFFu;
      float ds = d * (float)(byte & 15u);            // exact: 11 x 4 bits
      float mn = dmin * (float)(byte >> 4);          // exact
#pragma unroll
      for (int i = 0; i < 16; i++) {
        uint32_t qv = (q[i >> 2] >> (8 * (i & 3) + 2 * p)) & 3u;
        out[16 * p + i] = __builtin_fmaf(ds, (float)qv, -mn);  // one rounding
      }
    }
  }
  __device__ static int out_col(int ch, int j) { return seg_base(ch, j >> 4) + (j & 15); }
};

// IQ2_XXS: chunk = two 32-weight sub-blocks (a0, a1) of a superblock, weights
// 64c .. 64c + 63 of it; side = the superblock's fp16 d. The codebook (as bf16
// pairs) and the 128 sign masks (bits 15 and 31 of four words) live in LDS.
// The four bf16-pair sign masks of one IQ2_XXS group from its 7-bit sign code c:
// the 8-bit mask m is c plus its parity bit (an even number of negatives); word k
// carries m bit 2k at bit 15 and m bit 2k + 1 at bit 31. With Y = m << 15 | m << 30
// as a 64-bit value (two copies that do not overlap), word k is bits [2k, 2k + 32)
// of Y, masked to 0x80008000.
__device__ __forceinline__ void iq2_sign_words(uint32_t c, uint32_t* w) {
  const uint32_t m = c | ((uint32_t)(__builtin_popcount(c) & 1) << 7);
  const uint32_t ylo = (m << 15) | (m << 30), yhi = m >> 2;
#pragma unroll
  for (int k = 0; k < 4; k++) w[k] = __builtin_amdgcn_alignbit(yhi, ylo, 2 * k) & 0x80008000u;
}
__device__ __forceinline__ void iq2_fill_lds(Iq2Lds* t, const uint8_t* grid, int tid, int nthreads) {
  for (int i = tid; i < 256 * 4; i += nthreads) {
    uint32_t g0 = grid[2 * i], g1 = grid[2 * i + 1];
    t->grid[i] = (f32_bf16_rne((float)g0)) | (f32_bf16_rne((float)g1) << 16);
  }
  for (int c = tid; c < 128; c += nthreads) {
    uint32_t m[4];
    iq2_sign_words((uint32_t)c, m);
    t->sgn[c] = u32x4{m[0], m[1], m[2], m[3]};
  }
}
// The same table in two halves, for a 256-thread work-group that should not wait
// for the codebook before issuing its other loads: thread tid loads codebook entry
// tid (8 bytes) first, and stores it once those loads are in flight.
struct Iq2Entry {
  uint32_t b[8];
};
__device__ __forceinline__ Iq2Entry iq2_load_entry(const uint8_t* grid, int tid) {
  Iq2Entry e;
#pragma unroll
  for (int j = 0; j < 8; j++) e.b[j] = grid[8 * tid + j];
  return e;
}
__device__ __forceinline__ void iq2_store_entry(Iq2Lds* t, const Iq2Entry& e, int tid) {
#pragma unroll
  for (int k = 0; k < 4; k++)
    t->grid[4 * tid + k] = f32_bf16_rne((float)e.b[2 * k]) | (f32_bf16_rne((float)e.b[2 * k + 1]) << 16);
#if MOEQ_IQ2_SIGN_LDS
  if (tid < 128) {
    uint32_t m[4];
    iq2_sign_words((uint32_t)tid, m);
    t->sgn[tid] = u32x4{m[0], m[1], m[2], m[3]};
  }
#endif
}

template <> struct Dec<FMT_IQ2_XXS> {
  static constexpr int WPC = 64;
  typedef uint32_t Side;
  __device__ static Side side(const WView& w, int r, int ch) {
    return *reinterpret_cast<const uint16_t*>(w.scales + ((size_t)r * (w.cols / 256) + (ch >> 2)) * 2);
  }
  __device__ static const uint8_t* chunk_ptr(const WView& w, int r, int ch) {
    return w.data + (size_t)r * (w.cols / 256) * 64 + (size_t)ch * 16;
  }
  template <int ACT>
  __device__ static void fetch_x(const void* row, int ch, u32x4* raw) {
    Act<ACT>::template fetch<64>(row, ch * 64, raw);
  }
  template <int ACT>
  __device__ static void prep_x(const u32x4* raw, uint32_t* x, float*) {
    Act<ACT>::template from_raw<64>(raw, x);
  }
  template <int ACT>
  __device__ static void load_x(const void* row, int ch, uint32_t* x, float*) {
    Act<ACT>::template load<64>(row, ch * 64, x);
  }
  template <int ACT>
  __device__ static float dot(u32x4 q, Side s, const uint32_t* x, const float*, float acc, const Iq2Lds* t) {
    float d8 = half_bits_f32(s) * 0.125f;
#pragma unroll
    for (int j = 0; j < 2; j++) {
      uint32_t a0 = q[2 * j], a1 = q[2 * j + 1];
      float S = 0.f;
#pragma unroll
      for (int l = 0; l < 4; l++) {
        uint32_t gi = (a0 >> (8 * l)) & 0xFFu;
        uint32_t c = (a1 >> (7 * l)) & 0x7Fu;
        u32x4 g = *reinterpret_cast<const u32x4*>(&t->grid[gi * 4]);
#if MOEQ_IQ2_SIGN_LDS
        const u32x4 mv = t->sgn[c];
        const uint32_t m[4] = {mv[0], mv[1], mv[2], mv[3]};
#else
        // In registers: the GEMV is bound by its codebook reads from LDS and the VALU
        // together, and a second LDS read per group (the sign table) cost more than
        // the ten VALU operations it saves (bs=1 IQ2_XXS + Q2_K layer 27.4 against
        // 26.8 us).
        uint32_t m[4];
        iq2_sign_words(c, m);
#endif
        // sign bits of the codebook words are clear, so OR applies the signs
#pragma unroll
        for (int k = 0; k < 4; k++) S = dotp<ACT, 64>(g[k] | m[k], x, 16 * j + 4 * l + k, S);
      }
      float db = d8 * (float)(2u * (a1 >> 28) + 1u);
      acc = __builtin_fmaf(db, S, acc);
    }
    return acc;
  }
  __device__ static void to_f32(u32x4 q, Side s, float, const uint8_t* grid, float* out) {
    float d8 = half_bits_f32(s) * 0.125f;
#pragma unroll
    for (int j = 0; j < 2; j++) {
      uint32_t a0 = q[2 * j], a1 = q[2 * j + 1];
      float db = d8 * (float)(2u * (a1 >> 28) + 1u);  // exact: 11 x 5 bits
#pragma unroll
      for (int l = 0; l < 4; l++) {
        uint32_t gi = (a0 >> (8 * l)) & 0xFFu;
        uint32_t c = (a1 >> (7 * l)) & 0x7Fu;
        uint32_t m = c | ((uint32_t)(__builtin_popcount(c) & 1) << 7);
#pragma unroll
        for (int k = 0; k < 8; k++) {
          float v = db * (float)grid[gi * 8 + k];  // exact: 16 x 8 bits
          out[32 * j + 8 * l + k] = ((m >> k) & 1u) ? -v : v;
        }
      }
    }
  }
  __device__ static int out_col(int ch, int j) { return ch * 64 + j; }
};

// FP8 block-128: chunk = 16 e4m3 codes; side = the 128x128 tile's e8m0 code.
template <> struct Dec<FMT_FP8_B128> {
  static constexpr int WPC = 16;
  typedef uint32_t Side;
  __device__ static Side side(const WView& w, int r, int ch) {
    return w.scales[(size_t)(r >> 7) * (w.cols / 128) + (ch >> 3)];
  }
  __device__ static const uint8_t* chunk_ptr(const WView& w, int r, int ch) {
    return w.data + (size_t)r * w.cols + (size_t)ch * 16;
  }
  template <int ACT>
  __device__ static void fetch_x(const void* row, int ch, u32x4* raw) {
    Act<ACT>::template fetch<16>(row, ch * 16, raw);
  }
  template <int ACT>
  __device__ static void prep_x(const u32x4* raw, uint32_t* x, float*) {
    Act<ACT>::template from_raw<16>(raw, x);
  }
  template <int ACT>
  __device__ static void load_x(const void* row, int ch, uint32_t* x, float*) {
    Act<ACT>::template load<16>(row, ch * 16, x);
  }
  template <int ACT>
  __device__ static float dot(u32x4 q, Side s, const uint32_t* x, const float*, float acc, const Iq2Lds*) {
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      p = dotp<ACT, 16>(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[i], 1.0f, false)), x,
                        2 * i, p);
      p = dotp<ACT, 16>(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[i], 1.0f, true)), x,
                        2 * i + 1, p);
    }
    return __builtin_fmaf(p, e8m0_f32(s), acc);
  }
  __device__ static void to_f32(u32x4 q, Side s, float, const uint8_t*, float* out) {
    int ex = (int)s - 127;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q[i], 1.0f, false);
      f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q[i], 1.0f, true);
      out[4 * i + 0] = __builtin_ldexpf(a.x, ex);
      out[4 * i + 1] = __builtin_ldexpf(a.y, ex);
      out[4 * i + 2] = __builtin_ldexpf(b.x, ex);
      out[4 * i + 3] = __builtin_ldexpf(b.y, ex);
    }
    if (s == 255u) {
#pragma unroll
      for (int j = 0; j < 16; j++) out[j] = __builtin_nanf("");
    }
  }
  __device__ static int out_col(int ch, int j) { return ch * 16 + j; }
};

// E4M3 weights with a power-of-two (e8m0) scale: FP8 block-32 (one scale per
// 32 x 32 tile), MXFP8 (one per 32 along a row) and MXFP8 in the pre-stored
// matrix-instruction order. Chunk = 16 codes, side = the e8m0 code of its scale.
// The pre-stored order keeps, per tile of 16 rows x 128 columns, lane L = n + 16g
// of the 16x16x128 block-scaled instruction together: 32 bytes (row n, columns
// 16g + [0, 16) then 64 + 16g + [0, 16) of the tile) at tile * 2048 + 32 L; and
// per 16 rows x 512 columns, the lane's four scale bytes (row n, 32-blocks
// 4j + g of the four 128-column tiles j) at 256 * group + 4 L.
template <int FMT> struct DecFp8 {
  static constexpr int WPC = 16;
  typedef uint32_t Side;
  __device__ static Side side(const WView& w, int r, int ch) {
    const int b = ch >> 1;  // the chunk's 32-block along the row
    if (FMT == FMT_FP8_B32) return w.scales[(size_t)(r >> 5) * (w.cols / 32) + b];
    if (FMT == FMT_MXFP8) return w.scales[(size_t)r * (w.cols / 32) + b];
    // tiled: 16-row tile rt, 512-column group b / 16, step j = (b / 4) % 4, g = b % 4
    const size_t grp = (size_t)(r >> 4) * (w.cols / 512) + (b >> 4);
    return w.scales[grp * 256 + 4 * ((r & 15) + 16 * (b & 3)) + ((b >> 2) & 3)];
  }
  __device__ static const uint8_t* chunk_ptr(const WView& w, int r, int ch) {
    if (FMT != FMT_MXFP8_TILED) return w.data + (size_t)r * w.cols + (size_t)ch * 16;
    const int kt = ch >> 3, p = ch & 7;  // 128-column tile, 16-byte piece within it
    const size_t tile = (size_t)(r >> 4) * (w.cols / 128) + kt;
    return w.data + tile * 2048 + 32 * ((r & 15) + 16 * (p & 3)) + 16 * (p >> 2);
  }
  template <int ACT>
  __device__ static void fetch_x(const void* row, int ch, u32x4* raw) {
    Act<ACT>::template fetch<16>(row, ch * 16, raw);
  }
  template <int ACT>
  __device__ static void prep_x(const u32x4* raw, uint32_t* x, float*) {
    Act<ACT>::template from_raw<16>(raw, x);
  }
  template <int ACT>
  __device__ static void load_x(const void* row, int ch, uint32_t* x, float*) {
    Act<ACT>::template load<16>(row, ch * 16, x);
  }
  template <int ACT>
  __device__ static float dot(u32x4 q, Side s, const uint32_t* x, const float*, float acc, const Iq2Lds*) {
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      p = dotp<ACT, 16>(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[i], 1.0f, false)), x,
                        2 * i, p);
      p = dotp<ACT, 16>(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[i], 1.0f, true)), x,
                        2 * i + 1, p);
    }
    return __builtin_fmaf(p, e8m0_f32(s), acc);
  }
  __device__ static void to_f32(u32x4 q, Side s, float, const uint8_t*, float* out) {
    int ex = (int)s - 127;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q[i], 1.0f, false);
      f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q[i], 1.0f, true);
      out[4 * i + 0] = __builtin_ldexpf(a.x, ex);
      out[4 * i + 1] = __builtin_ldexpf(a.y, ex);
      out[4 * i + 2] = __builtin_ldexpf(b.x, ex);
      out[4 * i + 3] = __builtin_ldexpf(b.y, ex);
    }
    if (s == 255u) {
#pragma unroll
      for (int j = 0; j < 16; j++) out[j] = __builtin_nanf("");
    }
  }
  __device__ static int out_col(int ch, int j) { return ch * 16 + j; }
};
template <> struct Dec<FMT_MXFP8> : DecFp8<FMT_MXFP8> {};
template <> struct Dec<FMT_FP8_B32> : DecFp8<FMT_FP8_B32> {};
template <> struct Dec<FMT_MXFP8_TILED> : DecFp8<FMT_MXFP8_TILED> {};

// e8m0 exponent of a 32-block with maximum a: the smallest 2^e with a / 2^e <= 448
// (e = p - 9 if the frexp mantissa of a is <= 0.875, else p - 8), clamped to the
// code range; zero or subnormal maxima give 0.
__device__ __forceinline__ uint32_t mx_block_exponent(float amax) {
  const uint32_t ab = f2u(amax);
  if (ab < 0x00800000u) return 0u;
  const int p = (int)(ab >> 23) - 126;
  const uint32_t frac = ab & 0x007FFFFFu;
  const int e = (frac <= 0x00600000u) ? p - 9 : p - 8;
  const int E = e + 127;
  return (uint32_t)(E < 0 ? 0 : (E > 254 ? 254 : E));
}

// Two E4M3 terms of 16 consecutive bf16 values (v0, v1: 8 values each), with the
// e8m0 scale of their 32-block shared with the neighbouring lane (lane ^ 1 holds
// the block's other half). All lanes of the wave must call it.
typedef short i16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void bf16_terms(u32x4 v0, u32x4 v1, uint32_t (&w)[2][4], uint32_t (&E)[2]) {
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
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, 64));
    E[term] = mx_block_exponent(amax);
    const float scale = u2f(E[term] << 23);  // the conversions' scale operand: 2^(E - 127)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const i16x2_t lo =
          __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2_t{0, 0}, x[4 * j], x[4 * j + 1], scale, false);
      const i16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, x[4 * j + 2], x[4 * j + 3], scale, true);
      w[term][j] = (amax == 0.f) ? 0u : __builtin_bit_cast(uint32_t, hi);
    }
    if (term == 0) {
#pragma unroll
      for (int j = 0; j < 4; j++) {  // residual x - hi, exact in fp32
        const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[0][j], scale, false);
        const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[0][j], scale, true);
        x[4 * j] -= a[0];
        x[4 * j + 1] -= a[1];
        x[4 * j + 2] -= b[0];
        x[4 * j + 3] -= b[1];
      }
    }
  }
}

// NT E4M3 terms of 16 consecutive fp32 values (v: 4 loads of 4 values), each term
// with its e8m0 scale per 32 shared with lane ^ 1; the residual after each term is
// exact in fp32 and each term carries four more significant bits, so three terms
// keep about 12 (the error of an element is at most 2^-12 of it plus 2^-25.8 of its
// block's maximum) and four about 16. store(term, codes[4], E) receives each term as
// soon as it is made. All lanes of the wave must call it.
template <int NT, class Store>
__device__ __forceinline__ void f32_terms_each(const u32x4 (&v)[4], Store&& store) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) x[4 * i + j] = u2f(v[i][j]);
#pragma unroll
  for (int term = 0; term < NT; term++) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 16; j++) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[j]));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, 64));
    const uint32_t E = mx_block_exponent(amax);
    const float scale = u2f(E << 23);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const i16x2_t lo =
          __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2_t{0, 0}, x[4 * j], x[4 * j + 1], scale, false);
      const i16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, x[4 * j + 2], x[4 * j + 3], scale, true);
      w[j] = (amax == 0.f) ? 0u : __builtin_bit_cast(uint32_t, hi);
    }
    store(term, w, E);
    if (term + 1 < NT) {
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
template <int NT>
__device__ __forceinline__ void f32_terms(const u32x4 (&v)[4], uint32_t (&w)[NT][4], uint32_t (&E)[NT]) {
  f32_terms_each<NT>(v, [&](int t, const uint32_t (&c)[4], uint32_t e) {
#pragma unroll
    for (int j = 0; j < 4; j++) w[t][j] = c[j];
    E[t] = e;
  });
}
__device__ __forceinline__ void f32_terms3(const u32x4 (&v)[4], uint32_t (&w)[3][4], uint32_t (&E)[3]) {
  f32_terms<3>(v, w, E);
}

// Registers of one chunk's activation slice for a format and activation kind.
// 16-byte loads behind one chunk's activation slice (fetch_x / prep_x).
template <int FMT, int ACT> struct XRaw {
  static constexpr int N = RawN<ACT, Dec<FMT>::WPC>::V;
};
template <int FMT, int ACT> struct XRegs {
  static constexpr int N = Dec<FMT>::WPC / 2 * (ACT != ACT_BF16 ? 2 : 1);
  static constexpr int NS = (FMT == FMT_Q2_K) ? 4 : 1;
};

// -------------------------------------------------------------------------
// Reduction of NV values per lane over groups of `lpr` consecutive lanes
// (lpr a power of two <= 64). Halving exchanges first, so it costs about
// NV - 1 + log2(lpr / NV) exchanges instead of NV * log2(lpr). Afterwards lane
// l holds, in v[0 .. max(1, NV/lpr) - 1], the totals of value indices
// ((l % lpr) * NV) / lpr + i.
template <int NV>
__device__ __forceinline__ void group_reduce(float* v, int lpr, int lane) {
  int s = lpr >> 1;
#pragma unroll
  for (int h = NV / 2; h >= 1; h >>= 1) {
    if (s >= 1) {
      bool up = (lane & s) != 0;
#pragma unroll
      for (int i = 0; i < h; i++) {
        float keep = up ? v[i + h] : v[i];
        float send = up ? v[i] : v[i + h];
        v[i] = keep + __shfl_xor(send, s, 64);
      }
      s >>= 1;
    }
  }
  for (; s >= 1; s >>= 1) v[0] += __shfl_xor(v[0], s, 64);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  // silu(g) * u = g / (1 + e^-g) * u
  return __fdividef(g, 1.0f + __expf(-g)) * u;
}

}  // namespace moeq
