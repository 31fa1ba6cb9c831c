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
// kernel lists the 64-pair chunks of every expert. Each of the eight waves owns 32
// rows: for gate/up it streams the gate and the up rows of the same 32 features,
// which share every A fragment it reads (half the LDS reads per matrix
// instruction, and SwiGLU needs no exchange); for down one 32-row tile, which
// leaves registers for two work-groups per compute unit. K advances in chunks of 256 (eight 32-blocks): the
// chunk's A tile (64 token rows x 256 bytes, gathered through the routing
// permutation) is staged once in LDS, double-buffered, and shared by the eight
// waves; the weights go straight from HBM to registers one chunk ahead. Items
// with at most 32 pairs skip the second token tile's instructions.
//
// Order of K inside a chunk. The contraction is a sum, so any order of the eight
// 32-blocks is the same product as long as A, B and both scales follow it. The
// i-th instruction of a chunk (i = 0..3) takes blocks i and 4 + i as its two
// 32-wide halves. Then B lane (n, g) reads bytes [64g, 64g + 64) of the row's
// 128-byte chunk over the four instructions (four 16-byte loads from one 64-byte
// run) and its four scales are one aligned 32-bit word.
#include "moeq_device.h"
#include "moeq_kernels.h"

#include <mutex>

namespace moeq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned int u32x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int PF_KC = 256;                 // K per chunk
constexpr int PF_WAVES = 8;
constexpr int PF_THREADS = 64 * PF_WAVES;
constexpr int PF_PIECES = 1024 / PF_THREADS;  // 16-byte pieces of the A tile per thread
constexpr int PF_STRIDE = PF_KC + 16;      // LDS row of the A tile, padded by 16 bytes

// weight rows per work-group: 32 per wave (gate/up: 32 features, gate and up rows)
__host__ __device__ constexpr int pf_rows(bool) { return 32 * PF_WAVES; }

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

typedef int i32x4 __attribute__((ext_vector_type(4)));

// One chunk of a wave's weight tile: lane (n, g) holds bytes [64g, 64g + 64) of
// row n's 128-byte chunk.
struct BChunk {
  i32x4 q[4];
};

// Dynamic LDS of a work-group: the item's scales for all of K, staged once (rows
// padded by 16 bytes: a 32-lane read of one column then touches two rows per
// bank at most). A: [64 token rows][SP]; B: [NS][256 rows][SP], SP = cols/32 + 16.
__host__ __device__ constexpr int pf_scale_stride(int cols) { return cols / 32 + 16; }
__host__ __device__ constexpr int pf_weight_tiles(bool gate_up) { return gate_up ? 2 : 1; }
size_t pf_dynamic_lds(bool gate_up, int cols) {
  return (size_t)(PREFILL_MC + pf_weight_tiles(gate_up) * pf_rows(gate_up)) * pf_scale_stride(cols);
}

// down: 16 waves per compute unit (two work-groups), gate/up: what fits
template <bool GATE_UP>
__global__ __launch_bounds__(PF_THREADS) __attribute__((amdgpu_waves_per_eu(GATE_UP ? 1 : 4))) void k_prefill(
    PrefillParams P) {
  // weight tiles per wave: gate/up two (gate and up rows of the same features),
  // down one
  constexpr int NS = pf_weight_tiles(GATE_UP);
  constexpr int ROWS = pf_rows(GATE_UP);
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][PREFILL_MC][PF_STRIDE];
  __shared__ int pair_lds[PREFILL_MC];
  extern __shared__ __attribute__((aligned(16))) uint8_t pf_dyn[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = blockIdx.y;
  if (q >= P.route.n_chunks()[0]) return;  // whole work-group
  const int e = P.route.chunk_e()[q];
  const int pstart = P.route.offsets()[e] + P.route.chunk_m0()[q];
  const int M = min(PREFILL_MC, P.route.offsets()[e + 1] - pstart);
  const int nbase = blockIdx.x * ROWS;

  if (tid < PREFILL_MC) pair_lds[tid] = tid < M ? P.route.perm()[pstart + tid] : 0;
  __syncthreads();

  if (e >= P.n_experts) {  // bucket of out-of-range ids: outputs are zero
    for (int i = tid; i < M * ROWS; i += PF_THREADS) {
      const int m = i / ROWS, col = nbase + i % ROWS;
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
  const int nchunks = P.cols / PF_KC;
  const int ncw = P.cols / 128;  // 32-bit words of scales per row
  const int SP = pf_scale_stride(P.cols);
  const bool two_tiles = M > 32;
  const int n0 = nbase + wave * 32;  // this wave's 32 weight rows (gate/up: of both matrices)
  uint8_t* as_all = pf_dyn;
  uint8_t* bs_all = pf_dyn + PREFILL_MC * SP;
  const uint8_t* b_base[NS];
#pragma unroll
  for (int s = 0; s < NS; s++) b_base[s] = P.w[s].data + (size_t)e * P.w[s].estride;
  const uint32_t b_off = (uint32_t)(n0 + n) * (uint32_t)(P.cols / 2) + 64u * g;

  // Every load of the K loop is unconditional (token rows past M read pair 0's
  // row, chunks past the end re-read the last one): loads complete in issue order
  // and the compiler can then wait for exactly the oldest ones instead of draining
  // the queue. A pieces are 32-bit offsets from the uniform base (A has fewer
  // than 2^31 bytes, checked by the caller).
  uint32_t a_off[PF_PIECES];
  int a_dst[PF_PIECES];
#pragma unroll
  for (int j = 0; j < PF_PIECES; j++) {
    const int piece = tid + PF_THREADS * j;  // 0..1023
    const int r = piece >> 4, c16 = piece & 15;
    const int pr = pair_lds[r < M ? r : 0];
    const uint32_t arow = (uint32_t)(GATE_UP ? pr / P.top_k : pr);
    a_off[j] = arow * (uint32_t)P.cols + 16u * c16;
    a_dst[j] = r * PF_STRIDE + 16 * c16;
  }

  u32x4 a_pre[PF_PIECES];
  auto load_a = [&](int c) {
    c = min(c, nchunks - 1);
#pragma unroll
    for (int j = 0; j < PF_PIECES; j++) a_pre[j] = ld16(P.aq + a_off[j] + c * PF_KC);
  };
  auto load_b = [&](int c, BChunk (&b)[NS]) {
    c = min(c, nchunks - 1);
#pragma unroll
    for (int s = 0; s < NS; s++)
#pragma unroll
      for (int i = 0; i < 4; i++)
        b[s].q[i] = *reinterpret_cast<const i32x4*>(b_base[s] + b_off + c * (PF_KC / 2) + 16 * i);
  };
  // A fragment of K step i for token tile t from LDS buffer buf.
  auto read_a = [&](int buf, int i, int t) {
    const uint8_t* row = &a_lds[buf][32 * t + n][0];
    const u32x4 lo = *reinterpret_cast<const u32x4*>(row + 32 * i + 16 * g);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(row + 128 + 32 * i + 16 * g);
    return __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // the four scales of chunk c for this lane: token tile t (A), weight tile s (B)
  auto a_scales = [&](int c, int t) { return *reinterpret_cast<const uint32_t*>(as_all + (32 * t + n) * SP + 8 * c + 4 * g); };
  auto b_scales = [&](int c, int s) {
    return *reinterpret_cast<const uint32_t*>(bs_all + (s * ROWS + wave * 32 + n) * SP + 8 * c + 4 * g);
  };

  // Stage the scales of all of K, 8-byte pieces: the work-group's weight rows
  // (contiguous in the scale plane) and the item's token rows (gathered; rows
  // past M take pair 0's row, their results are never stored). The loads of a
  // batch are all issued, then the pipeline's first A and B loads, then the LDS
  // stores; the first stage's barrier publishes them.
  constexpr int SB = 32;  // pieces per thread per batch (one batch up to K = 4096)
  const int npr = P.cols / 256;  // 8-byte pieces per row
  const int nbp = NS * ROWS * npr, nap = PREFILL_MC * npr;
  auto scale_piece = [&](int i, const uint8_t*& src, uint8_t*& dst) {
    if (i < nbp) {
      const int s = i / (ROWS * npr), rem = i % (ROWS * npr), row = rem / npr, w8 = rem % npr;
      src = P.w[s].scales + (size_t)e * P.w[s].sestride + (size_t)(nbase + row) * (P.cols / 32) + 8 * w8;
      dst = bs_all + (s * ROWS + row) * SP + 8 * w8;
    } else {
      const int j = i - nbp, r = j / npr, w8 = j % npr;
      const int pr = pair_lds[r < M ? r : 0];
      const size_t arow = (size_t)(GATE_UP ? pr / P.top_k : pr);
      src = P.as + arow * (P.cols / 32) + 8 * w8;
      dst = as_all + r * SP + 8 * w8;
    }
  };
  bool started = false;
  for (int base = 0; base < nbp + nap; base += SB * PF_THREADS) {
    uint2 v[SB];
#pragma unroll
    for (int j = 0; j < SB; j++) {
      const int i = base + j * PF_THREADS + tid;
      if (i < nbp + nap) {
        const uint8_t* src;
        uint8_t* dst;
        scale_piece(i, src, dst);
        v[j] = *reinterpret_cast<const uint2*>(src);
      }
    }
    if (!started) {
      load_a(0);
      started = true;
    }
#pragma unroll
    for (int j = 0; j < SB; j++) {
      const int i = base + j * PF_THREADS + tid;
      if (i < nbp + nap) {
        const uint8_t* src;
        uint8_t* dst;
        scale_piece(i, src, dst);
        *reinterpret_cast<uint2*>(dst) = v[j];
      }
    }
  }

  v16f acc[NS][2];  // [weight tile][token tile]
#pragma unroll
  for (int s = 0; s < NS; s++)
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[s][t][r] = 0.f;

  // One chunk: publish A(c) in LDS, prefetch A(c + 1) then B(c + 1) (in that
  // order, so waiting for A never waits for the newer B), then the four K steps
  // on B(c). A stage past the last chunk only keeps the pipeline's shape.
  auto stage = [&](int c, const BChunk (&cur)[NS], BChunk (&pre)[NS]) {
    const int buf = c & 1;
#pragma unroll
    for (int j = 0; j < PF_PIECES; j++) *reinterpret_cast<u32x4*>(&a_lds[buf][0][0] + a_dst[j]) = a_pre[j];
    __syncthreads();
    load_a(c + 1);
    load_b(c + 1, pre);
    // keep the next stage's LDS stores (which wait for A(c + 1)) out of this
    // stage's matrix instructions
    __builtin_amdgcn_sched_barrier(0);
    if (c >= nchunks) return;
    uint32_t sb[NS];
#pragma unroll
    for (int s = 0; s < NS; s++) sb[s] = b_scales(c, s);
    const uint32_t sa0 = a_scales(c, 0);
    if (NS == 1) {
      // one weight tile: fragments read just before use (registers for two
      // work-groups per compute unit)
      if (two_tiles) {
        const uint32_t sa1 = a_scales(c, 1);
#pragma unroll
        for (int i = 0; i < 4; i++) {
          // an e2m1 operand occupies the low four registers of the tuple; the
          // instruction does not read the upper four
          const v8i b = __builtin_shufflevector(cur[0].q[i], cur[0].q[i], 0, 1, 2, 3, -1, -1, -1, -1);
          acc[0][0] = mfma_fp8_fp4(read_a(buf, i, 0), b, acc[0][0], byte_of(sa0, i), byte_of(sb[0], i));
          acc[0][1] = mfma_fp8_fp4(read_a(buf, i, 1), b, acc[0][1], byte_of(sa1, i), byte_of(sb[0], i));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const v8i b = __builtin_shufflevector(cur[0].q[i], cur[0].q[i], 0, 1, 2, 3, -1, -1, -1, -1);
          acc[0][0] = mfma_fp8_fp4(read_a(buf, i, 0), b, acc[0][0], byte_of(sa0, i), byte_of(sb[0], i));
        }
      }
    } else if (two_tiles) {
      // two weight tiles share each fragment; step i + 1's fragments are read
      // while step i's matrix instructions run
      const uint32_t sa1 = a_scales(c, 1);
      v8i a0 = read_a(buf, 0, 0), a1 = read_a(buf, 0, 1);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        v8i n0_ = a0, n1_ = a1;
        if (i < 3) {
          n0_ = read_a(buf, i + 1, 0);
          n1_ = read_a(buf, i + 1, 1);
        }
#pragma unroll
        for (int s = 0; s < NS; s++) {
          const v8i b = __builtin_shufflevector(cur[s].q[i], cur[s].q[i], 0, 1, 2, 3, -1, -1, -1, -1);
          acc[s][0] = mfma_fp8_fp4(a0, b, acc[s][0], byte_of(sa0, i), byte_of(sb[s], i));
          acc[s][1] = mfma_fp8_fp4(a1, b, acc[s][1], byte_of(sa1, i), byte_of(sb[s], i));
        }
        a0 = n0_;
        a1 = n1_;
      }
      // issue order: scale words and step 0's fragments, then per step the next
      // step's four LDS reads ahead of the step's matrix instructions
      __builtin_amdgcn_sched_group_barrier(0x100, 4 + NS + 2, 0);
#pragma unroll
      for (int i = 0; i < 3; i++) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NS, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NS, 0);
    } else {
      v8i a0 = read_a(buf, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        v8i n0_ = a0;
        if (i < 3) n0_ = read_a(buf, i + 1, 0);
#pragma unroll
        for (int s = 0; s < NS; s++) {
          const v8i b = __builtin_shufflevector(cur[s].q[i], cur[s].q[i], 0, 1, 2, 3, -1, -1, -1, -1);
          acc[s][0] = mfma_fp8_fp4(a0, b, acc[s][0], byte_of(sa0, i), byte_of(sb[s], i));
        }
        a0 = n0_;
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 + NS + 1, 0);
#pragma unroll
      for (int i = 0; i < 3; i++) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NS, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NS, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  __builtin_amdgcn_sched_barrier(0);  // A(0) (issued with the scales) before B(0)
  BChunk b0[NS], b1[NS];
  load_b(0, b0);
  for (int c = 0; c < nchunks; c += 2) {
    stage(c, b0, b1);
    stage(c + 1, b1, b0);
  }

  // epilogue
  const int mt = two_tiles ? 2 : 1;
#pragma unroll
  for (int t = 0; t < 2; t++) {
    if (t >= mt) continue;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int m = 32 * t + (r & 3) + 8 * (r >> 2) + 4 * g;
      const bool live = m < M;
      const size_t pair = (size_t)pair_lds[m];
      if (GATE_UP) {
        const float hv = silu_mul(acc[0][t][r], acc[NS - 1][t][r]);
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
      } else if (live) {
        P.partial[pair * P.rows + n0 + n] = acc[0][t][r] * P.rw[pair];
      }
    }
  }
}

bool prefill_fits(bool gate_up, int cols) {
  return pf_dynamic_lds(gate_up, cols) + 2 * PREFILL_MC * PF_STRIDE + 4 * PREFILL_MC <= 160 * 1024;
}

hipError_t launch_prefill(bool gate_up, const PrefillParams& p, int /*n_slots*/, hipStream_t s) {
  // rows and cols are multiples of 256 and the scales fit in LDS (checked by the caller)
  static std::once_flag lds_once;
  static hipError_t lds_rc = hipSuccess;
  std::call_once(lds_once, [] {
    // allow the largest dynamic LDS the checks admit
    const int dyn = 160 * 1024 - (int)(2 * PREFILL_MC * PF_STRIDE + 4 * PREFILL_MC);
    lds_rc = hipFuncSetAttribute((const void*)k_prefill<true>, hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
    if (lds_rc == hipSuccess)
      lds_rc = hipFuncSetAttribute((const void*)k_prefill<false>, hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
  });
  if (lds_rc != hipSuccess) return lds_rc;
  const size_t dyn = pf_dynamic_lds(gate_up, p.cols);
  dim3 g((unsigned)(p.rows / pf_rows(gate_up)), (unsigned)RouteView::max_chunks(p.route.E, p.route.P)), b(PF_THREADS);
  if (gate_up) hipLaunchKernelGGL(k_prefill<true>, g, b, dyn, s, p);
  else hipLaunchKernelGGL(k_prefill<false>, g, b, dyn, s, p);
  return hipGetLastError();
}

}  // namespace moeq
