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
// Schedule. A work item is (64 pairs of one expert, 256 weight rows); the route
// kernel lists the 64-pair chunks of every expert. The work-group's eight waves
// each own 32 weight rows. K advances in chunks of 256 (eight 32-blocks): the
// chunk's A tile (64 token rows x 256 bytes, gathered through the routing
// permutation) is staged once in LDS, double-buffered, and shared by the eight
// waves; the weights go straight from HBM to registers, one chunk ahead.
//
// Order of K inside a chunk. The contraction is a sum, so any order of the eight
// 32-blocks is the same product as long as A, B and both scales follow it. The
// i-th instruction of a chunk (i = 0..3) takes blocks i and 4 + i as its two
// 32-wide halves. Then B lane (n, g) reads bytes [64g, 64g + 64) of the row's
// 128-byte chunk over the four instructions (four 16-byte loads from one 64-byte
// run) and its four scales are one aligned 32-bit word.
#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int PF_KC = 256;                 // K per chunk
constexpr int PF_WAVES = 8;
constexpr int PF_ROWS = 32 * PF_WAVES;     // weight rows per work-group
constexpr int PF_THREADS = 64 * PF_WAVES;
constexpr int PF_STRIDE = PF_KC + 16;      // LDS row of the A tile, padded by 16 bytes

__device__ __forceinline__ v16f mfma_fp8_fp4(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0 /*A: fp8 e4m3*/, 4 /*B: fp4 e2m1*/, 0, sa, 0,
                                                         sb);
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

__device__ __forceinline__ int byte_of(uint32_t w, int i) { return (int)((w >> (8 * i)) & 0xFFu); }

template <bool GATE_UP>
__global__ __launch_bounds__(PF_THREADS) void k_prefill(PrefillParams P) {
  constexpr int NM = GATE_UP ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][PREFILL_MC][PF_STRIDE];
  __shared__ uint32_t as_lds[2][PREFILL_MC][2];
  __shared__ int pair_lds[PREFILL_MC];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = blockIdx.y;
  if (q >= P.route.n_chunks()[0]) return;  // whole work-group
  const int e = P.route.chunk_e()[q];
  const int pstart = P.route.offsets()[e] + P.route.chunk_m0()[q];
  const int M = min(PREFILL_MC, P.route.offsets()[e + 1] - pstart);
  const int nbase = blockIdx.x * PF_ROWS;

  if (tid < PREFILL_MC) pair_lds[tid] = tid < M ? P.route.perm()[pstart + tid] : 0;
  __syncthreads();

  if (e >= P.n_experts) {  // bucket of out-of-range ids: outputs are zero
    for (int i = tid; i < M * PF_ROWS; i += PF_THREADS) {
      const int m = i / PF_ROWS, col = nbase + i % PF_ROWS;
      const size_t pair = (size_t)pair_lds[m];
      if (GATE_UP) {
        P.hq[pair * P.rows + col] = 0;
        if (P.h_f32) P.h_f32[pair * P.rows + col] = 0.f;
        if (col % 32 == 0) P.hs[pair * (P.rows / 32) + col / 32] = 0;
      } else {
        P.partial[pair * P.rows + col] = 0.f;
      }
    }
    return;
  }

  const int n = lane & 31, g = lane >> 5;
  const int n0 = nbase + wave * 32;  // this wave's 32 weight rows
  const int nchunks = P.cols / PF_KC;
  const int mt = M > 32 ? 2 : 1;     // token tiles in use

  // A sources: this thread's two 16-byte pieces of the chunk tile and, for
  // threads below 64, one row's eight scales.
  const uint8_t* a_src[2];
  int a_dst[2];
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int piece = tid + PF_THREADS * j;  // 0..1023
    const int r = piece >> 4, c16 = piece & 15;
    const int arow = GATE_UP ? pair_lds[r] / P.top_k : pair_lds[r];
    a_src[j] = r < M ? P.aq + (size_t)arow * P.cols + 16 * c16 : nullptr;
    a_dst[j] = r * PF_STRIDE + 16 * c16;
  }
  const uint8_t* as_src = nullptr;
  if (tid < M) {
    const int arow = GATE_UP ? pair_lds[tid] / P.top_k : pair_lds[tid];
    as_src = P.as + (size_t)arow * (P.cols / 32);
  }
  // B sources: row n0 + n, bytes [64g, 64g + 64) of each 128-byte chunk
  const uint8_t* b_src[NM];
  const uint8_t* bs_src[NM];
#pragma unroll
  for (int j = 0; j < NM; j++) {
    b_src[j] = P.w[j].data + (size_t)e * P.w[j].estride + (size_t)(n0 + n) * (P.cols / 2) + 64 * g;
    bs_src[j] = P.w[j].scales + (size_t)e * P.w[j].sestride + (size_t)(n0 + n) * (P.cols / 32) + 4 * g;
  }

  u32x4 a_pre[2];
  uint2 as_pre = make_uint2(0u, 0u);
  u32x4 b_pre[NM][4];
  uint32_t bs_pre[NM];
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int j = 0; j < 2; j++)
      if (a_src[j]) a_pre[j] = ld16(a_src[j] + (size_t)c * PF_KC);
    if (as_src) as_pre = *reinterpret_cast<const uint2*>(as_src + 8 * c);
#pragma unroll
    for (int j = 0; j < NM; j++) {
#pragma unroll
      for (int i = 0; i < 4; i++) b_pre[j][i] = ld16(b_src[j] + (size_t)c * (PF_KC / 2) + 16 * i);
      bs_pre[j] = *reinterpret_cast<const uint32_t*>(bs_src[j] + 8 * c);
    }
  };

  v16f acc[NM][2];
#pragma unroll
  for (int j = 0; j < NM; j++)
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[j][t][r] = 0.f;

  load_chunk(0);
  for (int c = 0; c < nchunks; c++) {
    const int buf = c & 1;
#pragma unroll
    for (int j = 0; j < 2; j++)
      if (a_src[j]) *reinterpret_cast<u32x4*>(&a_lds[buf][0][0] + a_dst[j]) = a_pre[j];
    if (as_src) {
      as_lds[buf][tid][0] = as_pre.x;
      as_lds[buf][tid][1] = as_pre.y;
    }
    __syncthreads();
    u32x4 b_cur[NM][4];
    uint32_t bs_cur[NM];
#pragma unroll
    for (int j = 0; j < NM; j++) {
      bs_cur[j] = bs_pre[j];
#pragma unroll
      for (int i = 0; i < 4; i++) b_cur[j][i] = b_pre[j][i];
    }
    if (c + 1 < nchunks) load_chunk(c + 1);

#pragma unroll
    for (int i = 0; i < 4; i++) {
      v8i b[NM];
#pragma unroll
      for (int j = 0; j < NM; j++) {
        b[j][0] = (int)b_cur[j][i][0];
        b[j][1] = (int)b_cur[j][i][1];
        b[j][2] = (int)b_cur[j][i][2];
        b[j][3] = (int)b_cur[j][i][3];
        b[j][4] = b[j][5] = b[j][6] = b[j][7] = 0;
      }
#pragma unroll
      for (int t = 0; t < 2; t++) {
        if (t < mt) {
          const uint8_t* row = &a_lds[buf][32 * t + n][0];
          const u32x4 lo = *reinterpret_cast<const u32x4*>(row + 32 * i + 16 * g);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(row + 128 + 32 * i + 16 * g);
          v8i a;
          a[0] = (int)lo[0];
          a[1] = (int)lo[1];
          a[2] = (int)lo[2];
          a[3] = (int)lo[3];
          a[4] = (int)hi[0];
          a[5] = (int)hi[1];
          a[6] = (int)hi[2];
          a[7] = (int)hi[3];
          const int sa = byte_of(as_lds[buf][32 * t + n][g], i);
#pragma unroll
          for (int j = 0; j < NM; j++) acc[j][t] = mfma_fp8_fp4(a, b[j], acc[j][t], sa, byte_of(bs_cur[j], i));
        }
      }
    }
  }

  // epilogue
#pragma unroll
  for (int t = 0; t < 2; t++) {
    if (t >= mt) continue;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int m = 32 * t + (r & 3) + 8 * (r >> 2) + 4 * g;
      const bool live = m < M;
      const size_t pair = (size_t)pair_lds[m];
      if (GATE_UP) {
        const float hv = silu_mul(acc[0][t][r], acc[1][t][r]);
        if (live && P.h_f32) P.h_f32[pair * P.rows + n0 + n] = hv;
        // MXFP8 over this tile's 32 features of row m: the 32 lanes of one half hold the row
        float amax = __builtin_fabsf(hv);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, o, 64));
        const uint32_t E = amax == 0.f ? 0u : mx_exponent(amax);
        const uint32_t code = amax == 0.f ? 0u : e4m3_code(__builtin_ldexpf(hv, 127 - (int)E));
        if (live) {
          P.hq[pair * P.rows + n0 + n] = (uint8_t)code;
          if (n == 0) P.hs[pair * (P.rows / 32) + n0 / 32] = (uint8_t)E;
        }
      } else {
        if (live) P.partial[pair * P.rows + n0 + n] = acc[0][t][r] * P.rw[pair];
      }
    }
  }
}

hipError_t launch_prefill(bool gate_up, const PrefillParams& p, int /*n_slots*/, hipStream_t s) {
  // rows and cols are multiples of 256 (checked by the caller)
  dim3 g((unsigned)(p.rows / PF_ROWS), (unsigned)RouteView::max_chunks(p.route.E, p.route.P)), b(PF_THREADS);
  if (gate_up) hipLaunchKernelGGL(k_prefill<true>, g, b, 0, s, p);
  else hipLaunchKernelGGL(k_prefill<false>, g, b, 0, s, p);
  return hipGetLastError();
}

}  // namespace moeq
