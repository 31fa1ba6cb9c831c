// W4A8 prefill: token-grouped expert GEMMs on the gfx950 block-scaled matrix
// instruction v_mfma_scale_f32_32x32x64_f8f6f4 (A = E4M3 activations, B = e2m1
// weights, one e8m0 scale per 32 along K on both sides, fp32 accumulate).
//
// The prefill numerics are fp4 weights times E4M3 activations with a dynamic
// activation scale (DeepSeekv4 Flash for 1x Spark forum thread, second post);
// tokens are grouped by expert and each expert's weights are read once for all of
// its tokens (the same thread, fourth post: expert-major schedule).
//
//   gate/up: for expert e with tokens M_e (rows of Xq), per 32-wide tile of the
//            intermediate axis: G and U tiles over K = hidden, h = silu(g) u,
//            then h quantised to MXFP8 along the intermediate axis (one e8m0 per
//            32 = exactly the tile) -> hq, hs (and h itself, optionally)
//   down:    per 32-wide tile of the hidden axis: Hq_e . D_e^T over K = inter,
//            route-weighted -> partial[pair][hidden], then the slot-order combine.
//
// Operand layout of the instruction (pinned on the device): B lane L holds
// column L%32 at K = 32(L/32) + [0,32) (16 bytes of a weight row, low nibble
// first) and the scale of that 32-block; A lane L holds row L%32 with bytes 0-15
// at K = 16(L/32) + [0,16) and bytes 16-31 at K = 32 + 16(L/32) + [0,16), and the
// scale of K-block L/32; C lane L register r is row (r%4) + 8(r/4) + 4(L/32),
// column L%32.
//
// A work-group is (expert slot, group of four 32-wide N-tiles); each wave owns one
// N-tile and streams its weight rows once, applying every 64-wide K step to up to
// MT token tiles held in accumulators; experts with more tokens take more passes
// (the repeated weight reads then come from the caches).
#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int PF_MT = 2;  // token tiles of 32 per pass

__device__ __forceinline__ v16f mfma_fp8_fp4(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0 /*A: fp8 e4m3*/, 4 /*B: fp4 e2m1*/, 0, sa, 0,
                                                         sb);
}

// A fragment of K step s for token row `row` (a byte row of length kbytes).
__device__ __forceinline__ v8i load_a(const uint8_t* row, int s, int g) {
  const u32x4 lo = ld16(row + 64 * s + 16 * g);
  const u32x4 hi = ld16(row + 64 * s + 32 + 16 * g);
  v8i a;
  a[0] = (int)lo[0];
  a[1] = (int)lo[1];
  a[2] = (int)lo[2];
  a[3] = (int)lo[3];
  a[4] = (int)hi[0];
  a[5] = (int)hi[1];
  a[6] = (int)hi[2];
  a[7] = (int)hi[3];
  return a;
}

__device__ __forceinline__ v8i load_b(const uint8_t* wrow, int s, int g) {
  const u32x4 q = ld16(wrow + 16 * (2 * s + g));
  v8i b;
  b[0] = (int)q[0];
  b[1] = (int)q[1];
  b[2] = (int)q[2];
  b[3] = (int)q[3];
  b[4] = b[5] = b[6] = b[7] = 0;
  return b;
}

// E4M3FN round-to-nearest-even of v (saturating, sign kept); same rule as the
// activation quantiser.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  uint32_t sign = (f2u(v) >> 24) & 0x80u;
  float a = __builtin_fabsf(v);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    int e = (int)((f2u(a) >> 23) & 0xFFu) - 127;
    uint32_t q = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));
    if (q == 16u) {
      e += 1;
      q = 8u;
    }
    code = ((uint32_t)(e + 7) << 3) | (q - 8u);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code | sign;
}

__device__ __forceinline__ uint32_t mx_exponent(float amax) {
  uint32_t ab = f2u(amax);
  if (ab < 0x00800000u) return 0u;
  int p = (int)(ab >> 23) - 126;
  uint32_t frac = ab & 0x007FFFFFu;
  int e = (frac <= 0x00600000u) ? p - 9 : p - 8;
  int Ei = e + 127;
  return (uint32_t)(Ei < 0 ? 0 : (Ei > 254 ? 254 : Ei));
}

template <bool GATE_UP>
__global__ __launch_bounds__(256) void k_prefill(PrefillParams P) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = blockIdx.y;
  if (slot >= P.route.n_slots()[0]) return;
  const int e = P.route.slots()[slot];
  const int pstart = P.route.offsets()[e];
  const int M = P.route.offsets()[e + 1] - pstart;
  const int n0 = (blockIdx.x * 4 + wave) * 32;  // this wave's N-tile
  const bool valid_e = e >= 0 && e < P.n_experts;
  const int n = lane & 31, g = lane >> 5;
  const int ksteps = P.cols / 64;

  if (!valid_e) {  // bucket of out-of-range ids: outputs are zero
    if (n0 < P.rows) {
      for (int m = g; m < M; m += 2) {
        const int pair = P.route.perm()[pstart + m];
        if (GATE_UP) {
          P.hq[(size_t)pair * P.rows + n0 + n] = 0;
          if (P.h_f32) P.h_f32[(size_t)pair * P.rows + n0 + n] = 0.f;
          if (n == 0) P.hs[(size_t)pair * (P.rows / 32) + n0 / 32] = 0;
        } else {
          P.partial[(size_t)pair * P.rows + n0 + n] = 0.f;
        }
      }
    }
    return;
  }
  if (n0 >= P.rows) return;

  constexpr int NM = GATE_UP ? 2 : 1;
  const uint8_t* wrow[NM];
  const uint8_t* wsc[NM];
#pragma unroll
  for (int j = 0; j < NM; j++) {
    wrow[j] = P.w[j].data + (size_t)e * P.w[j].estride + (size_t)(n0 + n) * (P.cols / 2);
    wsc[j] = P.w[j].scales + (size_t)e * P.w[j].sestride + (size_t)(n0 + n) * (P.cols / 32);
  }

  for (int mt0 = 0; mt0 < M; mt0 += 32 * PF_MT) {
    // token rows of this pass (lane's A row is m = lane % 32 of each tile)
    const uint8_t* arow[PF_MT];
    const uint8_t* asrow[PF_MT];
#pragma unroll
    for (int t = 0; t < PF_MT; t++) {
      int m = mt0 + 32 * t + n;
      if (m >= M) m = M - 1;  // rows past the end are computed on a real row and never stored
      const int pair = P.route.perm()[pstart + m];
      const int arow_idx = GATE_UP ? pair / P.top_k : pair;
      arow[t] = P.aq + (size_t)arow_idx * P.cols;
      asrow[t] = P.as + (size_t)arow_idx * (P.cols / 32);
    }
    v16f acc[NM][PF_MT];
#pragma unroll
    for (int j = 0; j < NM; j++)
#pragma unroll
      for (int t = 0; t < PF_MT; t++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[j][t][r] = 0.f;

    for (int s = 0; s < ksteps; s++) {
      v8i b[NM];
      int sb[NM];
#pragma unroll
      for (int j = 0; j < NM; j++) {
        b[j] = load_b(wrow[j], s, g);
        sb[j] = wsc[j][2 * s + g];
      }
#pragma unroll
      for (int t = 0; t < PF_MT; t++) {
        if (mt0 + 32 * t < M) {
          const v8i a = load_a(arow[t], s, g);
          const int sa = asrow[t][2 * s + g];
#pragma unroll
          for (int j = 0; j < NM; j++) acc[j][t] = mfma_fp8_fp4(a, b[j], acc[j][t], sa, sb[j]);
        }
      }
    }

    // epilogue
#pragma unroll
    for (int t = 0; t < PF_MT; t++) {
      if (mt0 + 32 * t >= M) continue;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = mt0 + 32 * t + (r & 3) + 8 * (r >> 2) + 4 * g;
        const bool live = m < M;
        const int pair = P.route.perm()[pstart + (live ? m : 0)];
        if (GATE_UP) {
          const float hv = silu_mul(acc[0][t][r], acc[1][t][r]);
          if (live && P.h_f32) P.h_f32[(size_t)pair * P.rows + n0 + n] = hv;
          // MXFP8 over this tile's 32 features of row m: lanes of one half share the row
          float amax = __builtin_fabsf(hv);
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, o, 64));
          const uint32_t E = amax == 0.f ? 0u : mx_exponent(amax);
          const uint32_t code = amax == 0.f ? 0u : e4m3_code(__builtin_ldexpf(hv, 127 - (int)E));
          if (live) {
            P.hq[(size_t)pair * P.rows + n0 + n] = (uint8_t)code;
            if (n == 0) P.hs[(size_t)pair * (P.rows / 32) + n0 / 32] = (uint8_t)E;
          }
        } else {
          if (live) P.partial[(size_t)pair * P.rows + n0 + n] = acc[0][t][r] * P.rw[pair];
        }
      }
    }
  }
}

hipError_t launch_prefill(bool gate_up, const PrefillParams& p, int n_slots, hipStream_t s) {
  dim3 g((unsigned)((p.rows + 127) / 128), (unsigned)n_slots), b(256);
  if (gate_up) hipLaunchKernelGGL(k_prefill<true>, g, b, 0, s, p);
  else hipLaunchKernelGGL(k_prefill<false>, g, b, 0, s, p);
  return hipGetLastError();
}

}  // namespace moeq
