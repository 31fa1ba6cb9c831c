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
// Schedule. A work item is (64 pairs of one expert, a tile of weight rows); the
// route kernel lists the 64-pair chunks of every expert. Each wave owns 32 rows:
// for gate/up it streams the gate and the up rows of the same 32 features, which
// share every A fragment it reads (half the LDS reads per matrix instruction, and
// SwiGLU needs no exchange); for down two 32-row tiles of the down matrix, 128
// rows apart, which share the A fragments the same way (with one tile per wave the
// A tile was as many bytes as the weights, and the layer took 911-916 against
// 891 us at T = 2048). Four waves make a work-group, two of which share a compute
// unit.
// K advances in chunks of 256 (eight 32-blocks): the chunk's A tile (64 token
// rows x 256 bytes, gathered through the routing permutation) is staged once in
// LDS, double-buffered, and shared by the group's waves; the weights go straight
// from HBM to registers one chunk ahead. Items with at most 32 pairs skip the
// second token tile's instructions.
//
// Order of K inside a chunk. The contraction is a sum, so any order of the eight
// 32-blocks is the same product as long as A, B and both scales follow it. The
// i-th instruction of a chunk (i = 0..3) takes blocks i and 4 + i as its two
// 32-wide halves. Then B lane (n, g) reads bytes [64g, 64g + 64) of the row's
// 128-byte chunk over the four instructions (four 16-byte loads from one 64-byte
// run) and its four scales are one aligned 32-bit word.
#include "moeq_device.h"
#include "moeq_kernels.h"

#include <type_traits>

namespace moeq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned int u32x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int PF_KC = 256;                 // K per chunk
// Waves per work-group: 4. Waves with two weight tiles need about 250 registers,
// so two groups share a compute unit; a one-tile down wave gets up to 168, three
// groups to a unit (at 128 the compiler spills loop-invariant addresses, and every
// reload waits for the whole load queue). Several independent groups per unit let
// one's prologue and epilogue overlap the others' weight streams.
__host__ __device__ constexpr int pf_waves(bool) { return 4; }
#ifndef MOEQ_PF_DN_TILES
#define MOEQ_PF_DN_TILES 2
#endif
// Weight tiles per wave: gate/up two (the gate and the up rows of the same 32
// features), down MOEQ_PF_DN_TILES (32-row tiles of the down matrix 128 rows apart).
__host__ __device__ constexpr int pf_weight_tiles(bool gate_up) { return gate_up ? 2 : MOEQ_PF_DN_TILES; }
__host__ __device__ constexpr int pf_waves_per_simd(bool gate_up) { return pf_weight_tiles(gate_up) == 2 ? 2 : 3; }
constexpr int PF_STRIDE = PF_KC + 16;      // LDS row of the A tile, padded by 16 bytes

// weight rows per tile set: 32 per wave (gate/up: 32 features, gate and up rows)
__host__ __device__ constexpr int pf_rows(bool gate_up) { return 32 * pf_waves(gate_up); }
// output columns a work-group covers: gate/up one tile set (its tiles are the two
// matrices), down one per weight tile (tile s is rows 128 s + [0, 128))
__host__ __device__ constexpr int pf_span(bool gate_up) { return gate_up ? pf_rows(true) : pf_rows(false) * MOEQ_PF_DN_TILES; }

__device__ __forceinline__ v16f mfma_fp8_fp4(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0 /*A: fp8 e4m3*/, 4 /*B: fp4 e2m1*/, 0, sa, 0,
                                                         sb);
}

typedef short i16x2 __attribute__((ext_vector_type(2)));

// E4M3FN codes of a and b, round to nearest even, saturating to 448 with the sign
// kept (the activation quantiser's rule). The hardware conversion rounds to
// nearest even and handles subnormals the same way; it differs only above 448,
// where it gives NaN, and the select restores saturation there. Under the scale
// that mx_exponent picks, finite inputs never exceed 448.
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  uint32_t w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2{0, 0}, a, b, 1.0f, false));
  if (!(__builtin_fabsf(a) <= 448.0f)) w = (w & 0xFF00u) | 0x7Eu | ((f2u(a) >> 24) & 0x80u);
  if (!(__builtin_fabsf(b) <= 448.0f)) w = (w & 0x00FFu) | ((0x7Eu | ((f2u(b) >> 24) & 0x80u)) << 8);
  return w;
}

// max of v and its partner under a lane permutation inside each 16-lane row
template <int CTRL>
__device__ __forceinline__ float max_dpp(float v) {
  return __builtin_fmaxf(v, u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(v), CTRL, 0xF, 0xF, false)));
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

// Raw buffer of a uniform base: loads take a 32-bit per-lane offset and a uniform
// offset (the address stays in scalar registers; no 64-bit per-lane pointers).
// 0x00020000 is the gfx9-family buffer descriptor format word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}

// One chunk of a wave's weight tile: lane (n, g) holds bytes [64g, 64g + 64) of
// row n's 128-byte chunk.
struct BChunk {
  i32x4 q[4];
};

// Scales are staged in groups of PF_SG chunks (8 bytes per row per chunk) in a
// two-slot LDS ring, loaded PF_SG stages ahead of use, so every scale line of
// HBM is requested once per group instead of once per chunk. Rows are padded to
// 36 bytes (nine words), so a 32-lane read of one word column is conflict-free.
constexpr int PF_SG = 4;
constexpr int PF_SROW = 8 * PF_SG + 4;

template <bool GATE_UP>
__global__ __launch_bounds__(64 * pf_waves(GATE_UP)) __attribute__((
    amdgpu_waves_per_eu(pf_waves_per_simd(GATE_UP)))) void k_prefill(
    PrefillParams P) {
  // weight tiles per wave: gate/up two (gate and up rows of the same features),
  // down one
  constexpr int NS = pf_weight_tiles(GATE_UP);
  constexpr int ROWS = pf_rows(GATE_UP);
  constexpr int PF_THREADS = 64 * pf_waves(GATE_UP);
  constexpr int PF_PIECES = 1024 / PF_THREADS;  // 16-byte pieces of the A tile per thread
  static_assert(PF_THREADS >= 256, "one A-scale piece (64 rows x 4 chunks) per thread");
  constexpr int NBP = NS * ROWS * PF_SG / PF_THREADS;  // weight-scale pieces per thread per group
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][PREFILL_MC][PF_STRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t bs_ring[2][NS * ROWS][PF_SROW];
  __shared__ __attribute__((aligned(16))) uint8_t as_ring[2][PREFILL_MC][PF_SROW];
  __shared__ int pair_lds[PREFILL_MC];
  __shared__ float rw_lds[PREFILL_MC];  // down: route weight of each pair of the item

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = blockIdx.y;
  if (q >= P.route.n_chunks()[0]) return;  // whole work-group
  const int e = P.route.chunk_e()[q];
  const int pstart = P.route.offsets()[e] + P.route.chunk_m0()[q];
  const int M = min(PREFILL_MC, P.route.offsets()[e + 1] - pstart);
  constexpr int SPAN = pf_span(GATE_UP);
  const int nbase = blockIdx.x * SPAN;

  if (tid < PREFILL_MC) pair_lds[tid] = tid < M ? P.route.perm()[pstart + tid] : 0;
  __syncthreads();

  if (e >= P.n_experts) {  // bucket of out-of-range ids: outputs are zero
    for (int i = tid; i < M * SPAN; i += PF_THREADS) {
      const int m = i / SPAN, col = nbase + i % SPAN;
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

  // down: thread tid < 64 fetches pair tid's route weight now and publishes it in
  // LDS only at the epilogue, so the load's latency hides behind the K loop
  float rw_mine = 0.f;
  if constexpr (!GATE_UP) {
    if (tid < PREFILL_MC) rw_mine = P.rw[pair_lds[tid]];
  }
  const int n = lane & 31, g = lane >> 5;
  const int nchunks = P.cols / PF_KC;
  const bool two_tiles = M > 32;
  const int n0 = nbase + wave * 32;  // this wave's 32 weight rows (gate/up: of both matrices)
  __amdgpu_buffer_rsrc_t b_buf[NS], bs_buf[NS];
#pragma unroll
  for (int s = 0; s < NS; s++) {
    b_buf[s] = raw_buffer(P.w[s].data + (size_t)e * P.w[s].estride);
    bs_buf[s] = raw_buffer(P.w[s].scales + (size_t)e * P.w[s].sestride);
  }
  const __amdgpu_buffer_rsrc_t a_buf = raw_buffer(P.aq), as_buf = raw_buffer(P.as);
  const uint32_t b_off = (uint32_t)(n0 + n) * (uint32_t)(P.cols / 2) + 64u * g;

  // Every load of the K loop is unconditional (token rows past M read pair 0's
  // row, chunks past the end re-read the last one): loads complete in issue order
  // and the compiler can then wait for exactly the oldest ones instead of draining
  // the queue. Per-lane parts are 32-bit offsets from uniform bases (A has fewer
  // than 2^31 bytes, checked by the caller).
  uint32_t a_off[PF_PIECES];
#pragma unroll
  for (int j = 0; j < PF_PIECES; j++) {
    const int piece = tid + PF_THREADS * j;  // 0..1023
    const int r = piece >> 4, c16 = piece & 15;
    const int pr = pair_lds[r < M ? r : 0];
    const uint32_t arow = (uint32_t)(GATE_UP ? pr / P.top_k : pr);
    a_off[j] = arow * (uint32_t)P.cols + 16u * c16;
  }
  // LDS place of A piece j (recomputed at each use: cheaper than a register)
  auto a_dst = [&](int j) {
    const int piece = tid + PF_THREADS * j;
    return (piece >> 4) * PF_STRIDE + 16 * (piece & 15);
  };
  // Scale pieces of this thread: weight piece j is (tile, row, chunk k of the
  // group) of i = tid + PF_THREADS j with k = i % PF_SG, row = (i / PF_SG) % ROWS and
  // tile = i / (PF_SG ROWS) = PF_THREADS j / (PF_SG ROWS), known per j; the A piece
  // is (token row, k) of tid mod 256 (threads 256 apart load and store the same piece).
  static_assert((PF_SG * ROWS) % PF_THREADS == 0, "a weight-scale piece's tile is fixed per j");
  const int sk = tid % PF_SG;
  uint32_t as_src;
  {
    const int r = (tid & 255) / PF_SG;
    const int pr = pair_lds[r < M ? r : 0];
    const uint32_t arow = (uint32_t)(GATE_UP ? pr / P.top_k : pr);
    as_src = arow * (uint32_t)(P.cols / 32);
  }

  u32x4 a_pre[PF_PIECES];
  uint2 bs_pre[NBP], as_pre;
  auto load_a = [&](int c) {
    c = min(c, nchunks - 1);
#pragma unroll
    for (int j = 0; j < PF_PIECES; j++) a_pre[j] = __builtin_amdgcn_raw_buffer_load_b128(a_buf, a_off[j], c * PF_KC, 0);
  };
  auto load_b = [&](int c, BChunk (&b)[NS]) {
    c = min(c, nchunks - 1);
#pragma unroll
    for (int s = 0; s < NS; s++)
#pragma unroll
      for (int i = 0; i < 4; i++)
        b[s].q[i] = __builtin_bit_cast(
            i32x4, __builtin_amdgcn_raw_buffer_load_b128(b_buf[s], b_off + 16 * i, c * (PF_KC / 2), 0));
  };
  // scales of group G (chunks PF_SG G ..): the chunk index is clamped per piece
  auto load_scales = [&](int G) {
    // chunk PF_SG G + min(sk, last - PF_SG G): uniform part in the scalar offset
    const int kk = 8 * min(sk, nchunks - 1 - PF_SG * G);
#pragma unroll
    for (int j = 0; j < NBP; j++) {
      const int i = tid + PF_THREADS * j;
      const int s = (PF_THREADS * j) / (PF_SG * ROWS);
      const int row = (i / PF_SG) % ROWS;
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(
          bs_buf[s], (uint32_t)(nbase + row) * (uint32_t)(P.cols / 32) + kk, 8 * PF_SG * G, 0);
      bs_pre[j] = make_uint2(v[0], v[1]);
    }
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(as_buf, as_src + kk, 8 * PF_SG * G, 0);
    as_pre = make_uint2(v[0], v[1]);
  };
  auto store_scales = [&](int G) {
    const int slot = G & 1;
#pragma unroll
    for (int j = 0; j < NBP; j++) {
      const int i = tid + PF_THREADS * j;
      const int s = (PF_THREADS * j) / (PF_SG * ROWS);
      const int row = (i / PF_SG) % ROWS;
      uint32_t* d = reinterpret_cast<uint32_t*>(&bs_ring[slot][s * ROWS + row][8 * sk]);
      d[0] = bs_pre[j].x;
      d[1] = bs_pre[j].y;
    }
    uint32_t* d = reinterpret_cast<uint32_t*>(&as_ring[slot][(tid & 255) / PF_SG][8 * sk]);
    d[0] = as_pre.x;  // threads 256 apart store the same piece, same value
    d[1] = as_pre.y;
  };
  // A fragment of K step i for token tile t from LDS buffer buf.
  auto read_a = [&](int buf, int i, int t) {
    const uint8_t* row = &a_lds[buf][32 * t + n][0];
    const u32x4 lo = *reinterpret_cast<const u32x4*>(row + 32 * i + 16 * g);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(row + 128 + 32 * i + 16 * g);
    return __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // the four scales of chunk c for this lane: token tile t (A), weight tile s (B)
  auto a_scales = [&](int c, int t) {
    return *reinterpret_cast<const uint32_t*>(&as_ring[(c / PF_SG) & 1][32 * t + n][8 * (c % PF_SG) + 4 * g]);
  };
  auto b_scales = [&](int c, int s) {
    return *reinterpret_cast<const uint32_t*>(
        &bs_ring[(c / PF_SG) & 1][s * ROWS + wave * 32 + n][8 * (c % PF_SG) + 4 * g]);
  };

  v16f acc[NS][2];  // [weight tile][token tile]
#pragma unroll
  for (int s = 0; s < NS; s++)
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[s][t][r] = 0.f;

  // One chunk: publish A(c) (and, two stages into a group, the next group's
  // scales) in LDS, prefetch A(c + 1) then B(c + 1) (in that order, so waiting for
  // A never waits for the newer B; at a group's first stage the next group's
  // scales follow), then the four K steps on B(c). A stage past the last chunk
  // only keeps the pipeline's shape. SC: 1 = issue the next group's scale loads,
  // 2 = store them.
  auto stage = [&](auto sc_tag, int c, const BChunk (&cur)[NS], BChunk (&pre)[NS]) {
    constexpr int SC = decltype(sc_tag)::value;
    const int buf = c & 1;
#pragma unroll
    for (int j = 0; j < PF_PIECES; j++) *reinterpret_cast<u32x4*>(&a_lds[buf][0][0] + a_dst(j)) = a_pre[j];
    if constexpr (SC == 2) store_scales(c / PF_SG + 1);
    __syncthreads();
    load_a(c + 1);
    load_b(c + 1, pre);
    if constexpr (SC == 1) load_scales(c / PF_SG + 1);
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
        // token tiles one after the other: one fragment live at a time
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            // an e2m1 operand occupies the low four registers of the tuple; the
            // instruction does not read the upper four
            const v8i b = __builtin_shufflevector(cur[0].q[i], cur[0].q[i], 0, 1, 2, 3, -1, -1, -1, -1);
            acc[0][t] = mfma_fp8_fp4(read_a(buf, i, t), b, acc[0][t], byte_of(t ? sa1 : sa0, i), byte_of(sb[0], i));
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

  // prologue: group 0's scales, A(0), B(0); then group 0's scales into LDS (the
  // first stage's barrier publishes them)
  load_scales(0);
  load_a(0);
  __builtin_amdgcn_sched_barrier(0);  // A(0) before B(0), as every stage issues A before B
  BChunk b0[NS], b1[NS];
  load_b(0, b0);
  store_scales(0);
  using none = std::integral_constant<int, 0>;
  using issue = std::integral_constant<int, 1>;
  using store = std::integral_constant<int, 2>;
  static_assert(PF_SG == 4, "the loop body below is one group of four stages");
  for (int c = 0; c < nchunks; c += PF_SG) {
    stage(issue{}, c, b0, b1);
    stage(none{}, c + 1, b1, b0);
    stage(store{}, c + 2, b0, b1);
    stage(none{}, c + 3, b1, b0);
  }

  // epilogue
  const int mt = two_tiles ? 2 : 1;
  if constexpr (GATE_UP) {
    // h = silu(g) u, then MXFP8 of each token row's 32 features of this tile. Row m's
    // 32 values are register r of the 32 lanes of one half: their maximum comes from
    // four in-row lane permutations (xor 1, xor 2, the 8-lane and the 16-lane
    // mirror) and one exchange between the half's two 16-lane rows. Each step runs
    // over all sixteen registers before the next, so the exchanges overlap. The
    // codes go out through raw buffer stores with 32-bit offsets (hq and hs hold
    // fewer than 2^31 bytes, checked by the caller); a row past the item's last
    // pair gets an offset past the buffer's range, which the hardware drops.
    const int xaddr = (lane ^ 16) << 2;
    const __amdgpu_buffer_rsrc_t hq_buf = raw_buffer(P.hq), hs_buf = raw_buffer(P.hs);
    constexpr uint32_t kDrop = 0x7FFFFFFFu;  // the descriptors' record count
#pragma unroll
    for (int t = 0; t < 2; t++) {
      if (t >= mt) continue;
      float hv[16], am[16];
      int pr[16];
#pragma unroll
      for (int r = 0; r < 16; r++) pr[r] = pair_lds[32 * t + (r & 3) + 8 * (r >> 2) + 4 * g];
#pragma unroll
      for (int r = 0; r < 16; r++) {
        // silu(g) u with the hardware reciprocal (about 1 ulp)
        const float gv = acc[0][t][r];
        hv[r] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * acc[NS - 1][t][r];
        am[r] = __builtin_fabsf(hv[r]);
      }
#pragma unroll
      for (int r = 0; r < 16; r++) am[r] = max_dpp<0xB1>(am[r]);   // quad_perm [1,0,3,2]
#pragma unroll
      for (int r = 0; r < 16; r++) am[r] = max_dpp<0x4E>(am[r]);   // quad_perm [2,3,0,1]
#pragma unroll
      for (int r = 0; r < 16; r++) am[r] = max_dpp<0x141>(am[r]);  // row_half_mirror
#pragma unroll
      for (int r = 0; r < 16; r++) am[r] = max_dpp<0x140>(am[r]);  // row_mirror
#pragma unroll
      for (int r = 0; r < 16; r++)
        am[r] = __builtin_fmaxf(am[r], u2f((uint32_t)__builtin_amdgcn_ds_bpermute(xaddr, (int)f2u(am[r]))));
      uint32_t E[16], code[16];
#pragma unroll
      for (int r = 0; r < 16; r++) E[r] = am[r] == 0.f ? 0u : mx_exponent(am[r]);
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const uint32_t w = e4m3_pair(__builtin_ldexpf(hv[r], 127 - (int)E[r]),
                                     __builtin_ldexpf(hv[r + 1], 127 - (int)E[r + 1]));
        code[r] = am[r] == 0.f ? 0u : (w & 0xFFu);
        code[r + 1] = am[r + 1] == 0.f ? 0u : ((w >> 8) & 0xFFu);
      }
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const bool live = 32 * t + (r & 3) + 8 * (r >> 2) + 4 * g < M;
        const uint32_t row = (uint32_t)pr[r];
        const uint32_t oq = live ? row * (uint32_t)P.rows + (uint32_t)(n0 + n) : kDrop;
        const uint32_t os = live && n == 0 ? row * (uint32_t)(P.rows / 32) + (uint32_t)(n0 / 32) : kDrop;
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code[r], hq_buf, oq, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)E[r], hs_buf, os, 0, 0);
      }
      if (P.h_f32) {
#pragma unroll
        for (int r = 0; r < 16; r++)
          if (32 * t + (r & 3) + 8 * (r >> 2) + 4 * g < M) P.h_f32[(size_t)pr[r] * P.rows + n0 + n] = hv[r];
      }
    }
  } else {
    if (tid < PREFILL_MC) rw_lds[tid] = rw_mine;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 2; t++) {
      if (t >= mt) continue;
      int pr[16];
      float w[16];
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = 32 * t + (r & 3) + 8 * (r >> 2) + 4 * g;
        pr[r] = pair_lds[m];
        w[r] = rw_lds[m];
      }
#pragma unroll
      for (int s = 0; s < NS; s++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          if (32 * t + (r & 3) + 8 * (r >> 2) + 4 * g < M)
            P.partial[(size_t)pr[r] * P.rows + n0 + ROWS * s + n] = acc[s][t][r] * w[r];
        }
    }
  }
}

hipError_t launch_prefill(bool gate_up, const PrefillParams& p, int /*n_slots*/, hipStream_t s) {
  // rows and cols are multiples of 256 (checked by the caller)
  dim3 g((unsigned)(p.rows / pf_span(gate_up)), (unsigned)RouteView::max_chunks(p.route.E, p.route.P)),
      b((unsigned)(64 * pf_waves(gate_up)));
  if (gate_up) hipLaunchKernelGGL(k_prefill<true>, g, b, 0, s, p);
  else hipLaunchKernelGGL(k_prefill<false>, g, b, 0, s, p);
  return hipGetLastError();
}

}  // namespace moeq
