// Q2_K down projection of one token per grid row (the single-token layer, and the
// direct path of a few tokens) on the block-scaled FP8 matrix instruction
// v_mfma_scale_f32_16x16x128_f8f6f4, with no weight decode beyond a shift and a
// mask per four weights.
//
// Q2_K (IQ2_XXS + Q2_K + FP8 hybrid card, format table; DeepSeek-V4.1-Flash mixed-Q2
// GGUF card, Recipe): a 256-weight superblock of 2-bit codes q with a 4-bit scale
// sc and a 4-bit min m per 16 weights and fp16 d, dmin per superblock; weight =
// d sc q - dmin m. A code zero-extended to a byte is an E4M3 subnormal, q 2^-9, so
// the crumbs of a 16-byte chunk become FP8 operand bytes with one shift and one
// mask per dword and plane, and a B scale of 2^9 makes them the exact integers q.
//
// Device layout of a row's superblock: 64 data bytes as four 16-byte chunks c; bits
// 2p..2p+1 of byte j of chunk c (c = 2 h + s) hold weight 128 h + 32 p + 16 s + j,
// so plane p of chunk c is the 16 weights of sub-block 8 h + 2 p + s in order. Its
// 20-byte scale record holds sc | m << 4 of the 16 sub-blocks, then d | dmin << 16.
//
// Operands. Lane (row n, group g) loads chunk g of row n's superblock and passes
// two planes as its 32 B bytes (p0 at K = 16 g + [0, 16), p1 at K = 64 + 16 g +
// [0, 16)). h (fp32) enters as four base-16 digits on a grid of each 16-value
// sub-block (h_digits below): integers of at most 32 in magnitude, exact E4M3
// values, each digit row with its own e8m0 scale. Inside one 32-wide scale block the
// instruction drops products more than 2^-13 below the block's largest (measured on
// the device; its sums across blocks are exact fp32), so floating E4M3 terms of h
// would keep only about 13 bits; with integer digits every product of a row is a
// multiple of one unit and at most 96 units, so each dot is exact and h keeps 17
// bits relative to its sub-block's maximum. A row 4 q + t carries digit t of the
// sub-block that lane group q supplies at one of those two K ranges and zeros
// elsewhere, so two instructions per B operand (one per plane) give output lane
// (n, q), registers t = 0..3, the four digit products of sub-block (chunk q, plane
// p) of row n: exactly the sub-block whose scale byte that lane holds. The lane
// sums the digits' products, multiplies by sc, and adds m times the sub-block's
// exact sum of h for the min term; d and dmin apply once per superblock.
//
// Work: a work-group takes 16 output rows for all routed slots of its token, two
// waves per slot (half of K each). Every wave issues its scale-record and weight
// loads before it converts h; the slots' partial sums are combined in LDS in slot
// order with the route weights.
#include <hip/hip_runtime.h>

#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

namespace {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int QD_TERMS = 4;                         // digits of h
constexpr int QD_KPARTS = 2;                        // waves per slot
constexpr int QD_SB = 4;                            // superblocks per wave
constexpr int QD_KMAX = 256 * QD_SB * QD_KPARTS;    // 2048
constexpr int QD_SLOTS = 6;                         // routed slots (top-6)
constexpr int QD_REC = 5;                           // dwords of a scale record
constexpr int QD_WREC = 16 * QD_SB * QD_REC;        // a wave's records: 320 dwords

// Four base-16 digits of 16 consecutive fp32 values (a Q2_K sub-block; v: 4 loads
// of 4 values) on a grid of their own. With M their largest magnitude and s the
// exponent with M / 2^s in [16, 32), digit t is an integer on the grid 2^(s - 4t):
// d_0 = rint(v / 2^s) if that is at most 16, else twice rint(v / 2^(s+1)) (E4M3
// holds every integer up to 16 but only even ones up to 32); then d_t =
// rint(r_t / 2^(s - 4t)) with r_(t+1) = r_t - d_t 2^(s - 4t) (exact in fp32). So
// |d_0| <= 32, |d_1| <= 16, |d_2|, |d_3| <= 8, every digit is an exact E4M3 value, and
// |v - sum_t d_t 2^(s - 4t)| <= 2^(s - 13) <= 2^-17 M. store(t, j, code) gets the E4M3
// codes of digit t of values 4j .. 4j + 3, scale(t, E) its e8m0 code E = s - 4t + 127
// (clamped at 0, where the grid only gets coarser for tiny M).
template <class Store, class Scale>
__device__ __forceinline__ void h_digits(const u32x4 (&v)[4], Store&& store, Scale&& scale) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) x[4 * i + j] = u2f(v[i][j]);
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 16; j++) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[j]));
  const int s = (int)((f2u(amax) >> 23) & 0xFFu) - 131;  // floor(log2 M) - 4 (zero or subnormal M: -131)
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const int st = max(s - 4 * t, -127);
    const float inv = u2f((uint32_t)(127 - st) << 23);  // 2^-st
    const float sc = e8m0_f32((uint32_t)(st + 127));     // 2^st
#pragma unroll
    for (int j = 0; j < 4; j++) {
      float d[4];
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const float q = x[4 * j + k] * inv;
        d[k] = __builtin_rintf(q);
        if (t == 0) d[k] = __builtin_fabsf(q) <= 16.f ? d[k] : 2.f * __builtin_rintf(0.5f * q);
        x[4 * j + k] = __builtin_fmaf(-d[k], sc, x[4 * j + k]);
      }
      const i16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2_t{0, 0}, d[0], d[1], 1.0f, false);
      const i16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, d[2], d[3], 1.0f, true);
      store(t, j, __builtin_bit_cast(uint32_t, hi));
    }
    scale(t, (uint32_t)(st + 127));
  }
}

struct QdStage {
  uint8_t code[QD_TERMS][QD_SLOTS * QD_KMAX];       // E4M3 codes of h's digits, [slot][k]
  uint8_t sc[QD_TERMS][QD_SLOTS * QD_KMAX / 16];    // their e8m0 per 16 (sub-block)
  float hsum[QD_SLOTS * QD_KMAX / 16];              // exact sub-block sums, [slot][superblock][chunk][plane]
  uint32_t rec[QD_SLOTS * QD_KPARTS][QD_WREC];      // each wave's scale records, [row][superblock][dword]
};

// MOEQ_DQ_WPE: a minimum of waves per SIMD for the register allocation (6 would fit
// two work-groups per CU in 80 VGPRs, but spills a weight chunk).
#ifndef MOEQ_DQ_WPE
#define MOEQ_DQ_WPE 0
#endif
#if MOEQ_DQ_WPE
#define QD_ATTR __attribute__((amdgpu_waves_per_eu(MOEQ_DQ_WPE)))
#else
#define QD_ATTR
#endif
__global__ __launch_bounds__(64 * QD_KPARTS * QD_SLOTS) QD_ATTR void k_down1_q2k(Down1Params P) {
  __shared__ QdStage st;
  __shared__ float red[QD_SLOTS * QD_KPARTS][16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = wave / QD_KPARTS, part = wave % QD_KPARTS;
  const int n0 = blockIdx.x * 16;
  const int K = P.cols;
  const int nsb = K / 256;
  // Token blockIdx.y: its slots' ids, route weights, h and y.
  const int32_t* ids = P.ids + (size_t)blockIdx.y * P.top_k;
  const float* rwt = P.rw + (size_t)blockIdx.y * P.top_k;
  const float* ht = P.h + (size_t)blockIdx.y * P.top_k * K;
  float* yt = P.y + (size_t)blockIdx.y * P.rows;
  const int e = ids[slot];
  const bool ok = e >= 0 && e < P.n_experts;

  // Route weights and h first (thread t converts values 16t .. 16t + 15 of the
  // slots' concatenated h, [top_k][K]; threads past the end re-read the last 16).
  const int total = P.top_k * K;
  const int v0i = min(16 * (int)threadIdx.x, total - 16);
  const float rwv = rwt[min(lane, P.top_k - 1)];
  const float* hp = ht + v0i;
  const u32x4 hv[4] = {ld16(hp), ld16(hp + 4), ld16(hp + 8), ld16(hp + 12)};
  __builtin_amdgcn_sched_barrier(0);

  // The wave's superblocks [s0, s0 + my_sb); past the end, loads re-read the last.
  const int spw = (nsb + QD_KPARTS - 1) / QD_KPARTS;
  const int s0 = part * spw;
  const int my_sb = max(0, min(spw, nsb - s0));
  const int ec = ok ? e : 0;
  // Scale records of rows n0 .. n0 + 15 for the wave's superblocks: dword
  // d = lane + 64 j is dword d % 5 of record (row d / 20, superblock (d / 5) % 4).
  const uint8_t* sbase = P.w.scales + (size_t)ec * P.w.sestride;
  uint32_t rv[QD_WREC / 64];
#pragma unroll
  for (int j = 0; j < QD_WREC / 64; j++) {
    const int d = lane + 64 * j;
    const int r = min(n0 + d / (QD_SB * QD_REC), P.rows - 1);
    const int sbg = min(s0 + (d / QD_REC) % QD_SB, nsb - 1);
    rv[j] = *reinterpret_cast<const uint32_t*>(sbase + ((size_t)r * nsb + sbg) * (4 * QD_REC) + 4 * (d % QD_REC));
  }
  const int n = lane & 15, g = lane >> 4;
  const int rn = min(n0 + n, P.rows - 1);
  const uint8_t* wd = P.w.data + (size_t)ec * P.w.estride + (size_t)rn * nsb * 64 + 16 * g;
  u32x4 q[QD_SB];
#pragma unroll
  for (int i = 0; i < QD_SB; i++) q[i] = ld16(wd + (size_t)min(s0 + min(i, max(my_sb - 1, 0)), nsb - 1) * 64);
  __builtin_amdgcn_sched_barrier(0);

  // h -> four digits and the exact sum of each 16-value sub-block.
  if (16 * (int)threadIdx.x < total) {
    h_digits(
        hv, [&](int t, int j, uint32_t w) { *reinterpret_cast<uint32_t*>(&st.code[t][v0i + 4 * j]) = w; },
        [&](int t, uint32_t E) { st.sc[t][v0i / 16] = (uint8_t)E; });
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) s += (u2f(hv[i][0]) + u2f(hv[i][1])) + (u2f(hv[i][2]) + u2f(hv[i][3]));
    // sub-block j of the slot (j = 16 sb + 8 h + 2 p + s) -> [sb][chunk 2 h + s][plane p]
    const int sl = v0i / K, j = (v0i % K) / 16;
    const int c = 2 * ((j >> 3) & 1) + (j & 1), p = (j >> 1) & 3;
    st.hsum[sl * (K / 16) + (j & ~15) + 4 * c + p] = s;
  }
#pragma unroll
  for (int j = 0; j < QD_WREC / 64; j++) st.rec[wave][lane + 64 * j] = rv[j];
  __syncthreads();

  const int hb = slot * K;
  const int t = n & 3, qa = n >> 2;  // A row n = 4 qa + t: term t of lane group qa's sub-block
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < QD_SB; i++) {
    if (i < my_sb) {
      const int sb = s0 + i;
      const uint32_t* rec = &st.rec[wave][(n * QD_SB + i) * QD_REC];
      const int hh = g >> 1, ss = g & 1;
      // sc | m << 4 of planes 0, 1 (bytes 0, 2) and 2, 3 (bytes 0, 2)
      const uint32_t sw[2] = {rec[2 * hh] >> (8 * ss), rec[2 * hh + 1] >> (8 * ss)};
      const uint32_t dd = rec[4];
      const f32x4_t hs = *reinterpret_cast<const f32x4_t*>(&st.hsum[slot * (K / 16) + 16 * sb + 4 * g]);
      float acc_s = 0.f, acc_m = 0.f;
#pragma unroll
      for (int pp = 0; pp < 2; pp++) {
        // registers 0-3: plane 2 pp of the chunk, 4-7: plane 2 pp + 1
        i32x8_t bv;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          bv[j] = (int32_t)((q[i][j] >> (4 * pp)) & 0x03030303u);
          bv[4 + j] = (int32_t)((q[i][j] >> (4 * pp + 2)) & 0x03030303u);
        }
#pragma unroll
        for (int half = 0; half < 2; half++) {
          const int p = 2 * pp + half;
          u32x4 a = u32x4{0u, 0u, 0u, 0u};
          int sa = 0;
          {
            const int pos = hb + 256 * sb + 128 * (qa >> 1) + 32 * p + 16 * (qa & 1);
            sa = st.sc[t][pos / 16];
            if (qa == g) a = *reinterpret_cast<const u32x4*>(&st.code[t][pos]);
          }
          const u32x4 z = u32x4{0u, 0u, 0u, 0u};
          const i32x8_t av = half == 0 ? __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a, z, 0, 1, 2, 3, 4, 5, 6, 7))
                                       : __builtin_bit_cast(i32x8_t, __builtin_shufflevector(z, a, 0, 1, 2, 3, 4, 5, 6, 7));
          // B scale 2^9: the E4M3 subnormal codes q become the integers q.
          const f32x4_t cr =
              __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, sa, 0, 136);
          const uint32_t sm = sw[pp] >> (16 * half);
          acc_s = __builtin_fmaf((float)(sm & 15u), (cr[0] + cr[1]) + (cr[2] + cr[3]), acc_s);
          acc_m = __builtin_fmaf((float)((sm >> 4) & 15u), hs[p], acc_m);
        }
      }
      acc = __builtin_fmaf(half_bits_f32(dd), acc_s, acc);
      acc = __builtin_fmaf(-half_bits_f32(dd >> 16), acc_m, acc);
    }
  }
  // Loads past the wave's last superblock are never used: let them land first.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // the four chunks of each superblock: lane groups of column n
  acc += __shfl_xor(acc, 16, 64);
  acc += __shfl_xor(acc, 32, 64);
  if (lane < 16) red[wave][lane] = ok ? acc : 0.f;
  __syncthreads();
  if (threadIdx.x < 16) {
    float y = 0.f;
    for (int k = 0; k < P.top_k; k++) {
      float pk = 0.f;
#pragma unroll
      for (int h = 0; h < QD_KPARTS; h++) pk += red[k * QD_KPARTS + h][threadIdx.x];
      y += pk * u2f(__builtin_amdgcn_readlane(f2u(rwv), k));
    }
    const int r = n0 + (int)threadIdx.x;
    if (r < P.rows) yt[r] = y;
  }
  if (!ok && blockIdx.x == 0 && lane == 0 && part == 0) atomicOr(P.err, 1u);
}

}  // namespace

// K a multiple of 256 up to 2048, at most 6 slots.
bool down1_q2k_fits(int rows, int cols, int top_k) {
  return rows > 0 && cols > 0 && cols % 256 == 0 && cols <= QD_KMAX && top_k >= 1 && top_k <= QD_SLOTS;
}

hipError_t launch_down1_q2k(const Down1Params& p, hipStream_t s) {
  if (!down1_q2k_fits(p.rows, p.cols, p.top_k)) return hipErrorInvalidValue;
  dim3 g((unsigned)((p.rows + 15) / 16), (unsigned)(p.T > 1 ? p.T : 1)), b((unsigned)(64 * QD_KPARTS * p.top_k));
  hipLaunchKernelGGL(k_down1_q2k, g, b, 0, s, p);
  return hipGetLastError();
}

}  // namespace moeq
