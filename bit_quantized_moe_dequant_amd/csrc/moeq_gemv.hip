// Fused dequantize + GEMV kernels for the decode path, and the dequant kernel.
//
// Layout of the work: every lane owns a fixed slice of the contraction axis (CPL
// chunks of one 128-bit load each, chunks lr, lr + lpr, ... of a row, so a wave's
// loads are contiguous), keeps the activation slice for that range in registers,
// and walks over weight rows; `lpr` lanes share a row (lpr = 64 when a row has at
// least 64 chunks). Partial sums are reduced across the lpr lanes with halving
// exchanges. Weight bytes are read exactly once from HBM per token group.
//
// Kernels:
//   k_gemv<..., EPI_SWIGLU>  gate and up rows of one expert together, h = silu(g) u
//                            (REAP K180 Mixed NVFP4 card, "Why this mix?": gate/up
//                            carry two thirds of the expert bytes in decode)
//   k_gemv<..., EPI_PARTIAL> down rows, route-weighted, one output row per pair
//   k_gemv<..., EPI_PLAIN>   dense linear (FP8 block-128 dense layers)
//   k_down1                  down rows for a single token: one wave per routed
//                            expert, top-k combine in LDS in slot order
//   k_dequant                exact weights to fp32
#include <hip/hip_ext.h>

#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

template <int FMT>
__device__ __forceinline__ WView expert_view(const WeightRef& w, int e, int rows, int cols) {
  WView v;
  v.data = w.data + (size_t)e * w.estride;
  v.scales = w.scales + (size_t)e * w.sestride;
  v.rows = rows;
  v.cols = cols;
  return v;
}

// ---------------------------------------------------------------- dequant
template <int FMT>
__global__ __launch_bounds__(256) void k_dequant(WeightRef w, const uint8_t* grid, int rows, int cols, int expert,
                                                 float* out) {
  using D = Dec<FMT>;
  const int chunks = cols / D::WPC;
  size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)rows * chunks) return;
  int r = (int)(idx / chunks), ch = (int)(idx % chunks);
  WView v = expert_view<FMT>(w, expert, rows, cols);
  u32x4 q = ld16(D::chunk_ptr(v, r, ch));
  typename D::Side s = D::side(v, r, ch);
  float s2 = (FMT == FMT_NVFP4) ? w.scale2[expert] : 1.0f;
  float o[D::WPC];
  D::to_f32(q, s, s2, grid, o);
  float* orow = out + (size_t)r * cols;
#pragma unroll
  for (int j = 0; j < D::WPC; j++) orow[D::out_col(ch, j)] = o[j];
}

// ---------------------------------------------------------------- GEMV
#ifndef MOEQ_GEMV_WPE
#define MOEQ_GEMV_WPE 2  // waves per SIMD the register budget must allow
#endif
// Waves per SIMD the register budget must allow: MOEQ_GEMV_WPE, and one more for
// the one-token Q2_K down partials, which stay unspilled at that budget and run
// 4-6% faster with it (NVFP4 + Q2_K at T = 16, IQ2_XXS + Q2_K at T = 64); every
// other variant measured slower or spilled at three.
__host__ __device__ constexpr int gemv_wpe(int fmt, int epi, int mt) {
  return (fmt == FMT_Q2_K && epi == EPI_PARTIAL && mt == 1) ? MOEQ_GEMV_WPE + 1 : MOEQ_GEMV_WPE;
}

template <int FMT, int CPL, int MT, int NMAT, int EPI, int ACT, int UB, int NB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(gemv_wpe(FMT, EPI, MT)))) void k_gemv(GemvParams P) {
  using D = Dec<FMT>;
  typedef typename D::Side Side;
  constexpr int XN = XRegs<FMT, ACT>::N;
  constexpr int XS = XRegs<FMT, ACT>::NS;
  constexpr int NV = UB * MT;
  __shared__ Iq2Lds lds_tab[FMT == FMT_IQ2_XXS ? 1 : 1];
  (void)lds_tab;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = blockIdx.y;
  const int lpr = P.lpr;
  const int rw_rows = 64 / lpr;  // rows per wave step
  const int lr = lane & (lpr - 1);
  const int rsub = lane / lpr;

  // Resolve the expert and its pairs.
  int e, M, pstart = 0;
  if (P.mode == MODE_DIRECT) {
    e = P.ids[slot];
    M = 1;
  } else if (P.mode == MODE_GROUPED) {
    if (slot >= P.route.n_slots()[0]) return;
    e = P.route.slots()[slot];
    pstart = P.route.offsets()[e];
    M = P.route.offsets()[e + 1] - pstart;
  } else {
    e = P.expert;
    M = P.T;
  }

  const int tile_r0 = blockIdx.x * P.rows_per_wg;
  const int wr0 = tile_r0 + wave * (P.U * rw_rows);
  const bool bad = (e < 0 || e >= P.n_experts);
  if (bad) {
    // Out-of-range expert id: its pairs contribute nothing. Zero their outputs.
    if (P.mode == MODE_DIRECT && threadIdx.x == 0 && blockIdx.x == 0) atomicOr(P.err, 1u);
    if (EPI != EPI_PLAIN) {
      for (int m = 0; m < M; m++) {
        int pair = (P.mode == MODE_DIRECT) ? slot : P.route.perm()[pstart + m];
        for (int r = tile_r0 + threadIdx.x; r < tile_r0 + P.rows_per_wg && r < P.rows; r += 256)
          P.out[(size_t)pair * P.rows + r] = 0.f;
      }
    }
    return;
  }

  // IQ2_XXS codebook: each thread's entry is requested before the activation and
  // weight loads and stored to LDS once they are in flight (first tile only), so
  // the weight stream does not wait for it.
  Iq2Entry gent;
  if constexpr (FMT == FMT_IQ2_XXS) gent = iq2_load_entry(P.grid, threadIdx.x);

  WView W[NMAT];
#pragma unroll
  for (int mt = 0; mt < NMAT; mt++) W[mt] = expert_view<FMT>(P.w[mt], e, P.rows, P.cols);
  float s2[NMAT];
#pragma unroll
  for (int mt = 0; mt < NMAT; mt++) s2[mt] = (FMT == FMT_NVFP4) ? P.w[mt].scale2[e] : 1.0f;

  constexpr int XR = XRaw<FMT, ACT>::N;
  for (int m0 = 0; m0 < M; m0 += MT) {
    // Loads go out in the order they are needed, all before any arithmetic: the
    // activation slices of the tile's tokens, then the weight rows batch by batch.
    // They complete in issue order, so the first batch's arithmetic overlaps the
    // later batches' transfer. Every load is unconditional: tokens past the
    // expert's last re-read its last token, rows and chunks past the end the last
    // valid one; their results are masked.
    u32x4 xraw[MT][CPL][XR];
#pragma unroll
    for (int mi = 0; mi < MT; mi++) {
      const int m = min(m0 + mi, M - 1);
      const int pair = (P.mode == MODE_DIRECT) ? slot : (P.mode == MODE_GROUPED ? P.route.perm()[pstart + m] : m);
      const void* row;
      if (ACT == ACT_BF16) {
        const int tok = (P.mode == MODE_LINEAR) ? m : pair / P.top_k;
        row = reinterpret_cast<const uint16_t*>(P.act) + (size_t)tok * P.cols;
      } else {
        row = reinterpret_cast<const float*>(P.act) + (size_t)pair * P.cols;
      }
#pragma unroll
      for (int c = 0; c < CPL; c++) D::template fetch_x<ACT>(row, min(lr + lpr * c, P.chunks - 1), xraw[mi][c]);
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4 q[NB][NMAT][UB][CPL];
    Side sd[NB][NMAT][UB][CPL];
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
      for (int mt = 0; mt < NMAT; mt++)
#pragma unroll
        for (int ub = 0; ub < UB; ub++) {
          const int r = min(wr0 + (nb * UB + ub) * rw_rows + rsub, P.rows - 1);
#pragma unroll
          for (int c = 0; c < CPL; c++) {
            const int ch = min(lr + lpr * c, P.chunks - 1);
            q[nb][mt][ub][c] = ld16(D::chunk_ptr(W[mt], r, ch));
            sd[nb][mt][ub][c] = D::side(W[mt], r, ch);
          }
        }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FMT == FMT_IQ2_XXS) {
      if (m0 == 0) {  // uniform
        iq2_store_entry(&lds_tab[0], gent, threadIdx.x);
        __syncthreads();
      }
    }
    uint32_t x[MT][CPL][XN];
    float xs[MT][CPL][XS];
#pragma unroll
    for (int mi = 0; mi < MT; mi++)
#pragma unroll
      for (int c = 0; c < CPL; c++) D::template prep_x<ACT>(xraw[mi][c], x[mi][c], xs[mi][c]);
    // Chunks past the row end contribute nothing: both operands are zeroed, the
    // activations here and the weights where they are used (a NaN code times a
    // zero activation would still be NaN; overwriting a load's destination here
    // would have to wait for the load).
    bool cvalid[CPL];
#pragma unroll
    for (int c = 0; c < CPL; c++) {
      cvalid[c] = lr + lpr * c < P.chunks;
      if (!cvalid[c]) {
#pragma unroll
        for (int mi = 0; mi < MT; mi++) {
#pragma unroll
          for (int j = 0; j < XN; j++) x[mi][c][j] = 0u;
#pragma unroll
          for (int j = 0; j < XS; j++) xs[mi][c][j] = 0.f;
        }
      }
    }

#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      const int u0 = nb * UB;
      float acc[NMAT][NV];
#pragma unroll
      for (int mt = 0; mt < NMAT; mt++)
#pragma unroll
        for (int ub = 0; ub < UB; ub++)
#pragma unroll
          for (int mi = 0; mi < MT; mi++) {
            float a = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; c++)
              a = D::template dot<ACT>(cvalid[c] ? q[nb][mt][ub][c] : u32x4{0u, 0u, 0u, 0u},
                                       cvalid[c] ? sd[nb][mt][ub][c] : Side{}, x[mi][c], xs[mi][c], a, &lds_tab[0]);
            acc[mt][ub * MT + mi] = a;
          }
#pragma unroll
      for (int mt = 0; mt < NMAT; mt++) group_reduce<NV>(acc[mt], lpr, lane);

      // Lane holds value indices vi0 + i, i < nf.
      const int nf = NV >= lpr ? NV / lpr : 1;
      const bool writer = NV >= lpr ? true : ((lr % (lpr / NV)) == 0);
      const int vi0 = (lr * NV) / lpr;
      if (writer) {
#pragma unroll
        for (int i = 0; i < NV; i++) {
          if (i < nf) {
            const int vi = vi0 + i;
            const int ub = vi / MT, mi = vi % MT;
            const int r = wr0 + (u0 + ub) * rw_rows + rsub;
            const int m = m0 + mi;
            if (r < P.rows && m < M) {
              int pair = (P.mode == MODE_DIRECT) ? slot : (P.mode == MODE_GROUPED ? P.route.perm()[pstart + m] : m);
              float v;
              if (EPI == EPI_SWIGLU) {
                v = silu_mul(acc[0][i] * s2[0], acc[NMAT - 1][i] * s2[NMAT - 1]);
              } else if (EPI == EPI_PARTIAL) {
                v = acc[0][i] * s2[0] * P.rw[pair];
              } else {
                v = acc[0][i] * s2[0];
              }
              P.out[(size_t)pair * P.rows + r] = v;
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- down for one token
// One wave per routed slot (top_k <= MAXW). The bound on the work-group size sets
// the register budget: MAXW = 8 leaves 256 VGPRs, enough to keep every load of a
// wave in flight for every format; MAXW = 16 leaves 128.
template <int FMT, int CPL, int UB, int NB, int MAXW>
__global__ __launch_bounds__(64 * MAXW) void k_down1(Down1Params P) {
  using D = Dec<FMT>;
  typedef typename D::Side Side;
  constexpr int XN = XRegs<FMT, ACT_F32>::N;
  constexpr int XS = XRegs<FMT, ACT_F32>::NS;
  __shared__ Iq2Lds lds_tab[1];
  __shared__ float red[MAXW][64];

  const int lane = threadIdx.x & 63;
  // Slot handled by this wave; uniform, so its expert id is a scalar load.
  const int k = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lpr = P.lpr;
  const int rw_rows = 64 / lpr;
  const int lr = lane & (lpr - 1);
  const int rsub = lane / lpr;
  const int tile_r0 = blockIdx.x * P.rows_per_wg;

  if constexpr (FMT == FMT_IQ2_XXS) {
    iq2_fill_lds(&lds_tab[0], P.grid, threadIdx.x, blockDim.x);
    __syncthreads();
  }

  const int e = P.ids[k];
  const bool ok = (e >= 0 && e < P.n_experts);
  if (!ok && lane == 0 && blockIdx.x == 0) atomicOr(P.err, 1u);
  if (ok) {
    WView W = expert_view<FMT>(P.w, e, P.rows, P.cols);
    const float s2 = (FMT == FMT_NVFP4) ? P.w.scale2[e] : 1.0f;
    const float wk = P.rw[k] * s2;
    // Loads go out in the order they are needed, all before any arithmetic: the h
    // slice, then the weights batch by batch. They complete in issue order, so the
    // first batch's arithmetic overlaps the later batches' transfer instead of
    // waiting for the wave's last byte. Every load is unconditional: rows and
    // chunks past the end re-read the last valid one and are masked afterwards.
    constexpr int XR = XRaw<FMT, ACT_F32>::N;
    const float* hrow = P.h + (size_t)k * P.cols;
    u32x4 hraw[CPL][XR];
#pragma unroll
    for (int c = 0; c < CPL; c++) D::template fetch_x<ACT_F32>(hrow, min(lr + lpr * c, P.chunks - 1), hraw[c]);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 q[NB][UB][CPL];
    Side sd[NB][UB][CPL];
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
      for (int ub = 0; ub < UB; ub++) {
        const int r = min(tile_r0 + (nb * UB + ub) * rw_rows + rsub, P.rows - 1);
#pragma unroll
        for (int c = 0; c < CPL; c++) {
          const int ch = min(lr + lpr * c, P.chunks - 1);
          q[nb][ub][c] = ld16(D::chunk_ptr(W, r, ch));
          sd[nb][ub][c] = D::side(W, r, ch);
        }
      }
    __builtin_amdgcn_sched_barrier(0);
    uint32_t x[CPL][XN];
    float xs[CPL][XS];
#pragma unroll
    for (int c = 0; c < CPL; c++) D::template prep_x<ACT_F32>(hraw[c], x[c], xs[c]);
    // Chunks past the row end contribute nothing: both operands are zeroed, the
    // activations here and the weights where they are used (a NaN code times a
    // zero activation would still be NaN; overwriting a load's destination here
    // would have to wait for the load).
    bool cvalid[CPL];
#pragma unroll
    for (int c = 0; c < CPL; c++) {
      cvalid[c] = lr + lpr * c < P.chunks;
      if (!cvalid[c]) {
#pragma unroll
        for (int j = 0; j < XN; j++) x[c][j] = 0u;
#pragma unroll
        for (int j = 0; j < XS; j++) xs[c][j] = 0.f;
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      const int u0 = nb * UB;
      float acc[UB];
#pragma unroll
      for (int ub = 0; ub < UB; ub++) {
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; c++)
          a = D::template dot<ACT_F32>(cvalid[c] ? q[nb][ub][c] : u32x4{0u, 0u, 0u, 0u},
                                       cvalid[c] ? sd[nb][ub][c] : Side{}, x[c], xs[c], a, &lds_tab[0]);
        acc[ub] = a;
      }
      group_reduce<UB>(acc, lpr, lane);
      const int nf = UB >= lpr ? UB / lpr : 1;
      const bool writer = UB >= lpr ? true : ((lr % (lpr / UB)) == 0);
      const int vi0 = (lr * UB) / lpr;
      if (writer) {
#pragma unroll
        for (int i = 0; i < UB; i++) {
          if (i < nf) {
            const int ub = vi0 + i;
            if (u0 + ub < P.U) red[k][(u0 + ub) * rw_rows + rsub] = acc[i] * wk;
          }
        }
      }
    }
  } else {
    for (int i = lane; i < P.rows_per_wg; i += 64) red[k][i] = 0.f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < P.rows_per_wg; i += blockDim.x) {
    const int r = tile_r0 + i;
    if (r < P.rows) {
      float y = 0.f;
      for (int kk = 0; kk < P.top_k; kk++) y += red[kk][i];
      P.y[r] = y;
    }
  }
}

// ---------------------------------------------------------------- launchers
int weights_per_chunk(int fmt) {
  switch (fmt) {
    case FMT_MXFP4: return 32;
    case FMT_NVFP4: return 32;
    case FMT_Q2_K: return 64;
    case FMT_IQ2_XXS: return 64;
    case FMT_FP8_B128: return 16;
    case FMT_MXFP8: return 16;
    case FMT_FP8_B32: return 16;
    case FMT_MXFP8_TILED: return 16;
  }
  return 0;
}

// lpr = lanes sharing a row (a power of two <= 64), cpl = chunks per lane (1, 2
// or 4); lanes whose chunk index falls past the row end are masked.
bool chunk_geometry(int fmt, int cols, int* lpr, int* cpl) {
  int wpc = weights_per_chunk(fmt);
  if (wpc == 0 || cols <= 0 || cols % wpc) return false;
  int chunks = cols / wpc;
  int l = 1;
  while (l < chunks && l < 64) l <<= 1;
  int c = (chunks + l - 1) / l;
  if (c == 3) c = 4;
  if (c > 4) return false;
  *lpr = l;
  *cpl = c;
  return true;
}

hipError_t launch_dequant(int fmt, const WeightRef& w, const uint8_t* grid, int rows, int cols, int expert, float* out,
                          hipStream_t s) {
  int wpc = weights_per_chunk(fmt);
  size_t n = (size_t)rows * (cols / wpc);
  dim3 grid_dim((unsigned)((n + 255) / 256)), blk(256);
  switch (fmt) {
    case FMT_MXFP4: hipLaunchKernelGGL(k_dequant<FMT_MXFP4>, grid_dim, blk, 0, s, w, grid, rows, cols, expert, out); break;
    case FMT_NVFP4: hipLaunchKernelGGL(k_dequant<FMT_NVFP4>, grid_dim, blk, 0, s, w, grid, rows, cols, expert, out); break;
    case FMT_Q2_K: hipLaunchKernelGGL(k_dequant<FMT_Q2_K>, grid_dim, blk, 0, s, w, grid, rows, cols, expert, out); break;
    case FMT_IQ2_XXS:
      hipLaunchKernelGGL(k_dequant<FMT_IQ2_XXS>, grid_dim, blk, 0, s, w, grid, rows, cols, expert, out);
      break;
    case FMT_FP8_B128:
      hipLaunchKernelGGL(k_dequant<FMT_FP8_B128>, grid_dim, blk, 0, s, w, grid, rows, cols, expert, out);
      break;
    case FMT_MXFP8: hipLaunchKernelGGL(k_dequant<FMT_MXFP8>, grid_dim, blk, 0, s, w, grid, rows, cols, expert, out); break;
    case FMT_FP8_B32:
      hipLaunchKernelGGL(k_dequant<FMT_FP8_B32>, grid_dim, blk, 0, s, w, grid, rows, cols, expert, out);
      break;
    case FMT_MXFP8_TILED:
      hipLaunchKernelGGL(k_dequant<FMT_MXFP8_TILED>, grid_dim, blk, 0, s, w, grid, rows, cols, expert, out);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

#ifndef MOEQ_GEMV_UB
#define MOEQ_GEMV_UB 4  // rows per batch (gate/up, linear, grouped down)
#endif
#ifndef MOEQ_GEMV_NB
#define MOEQ_GEMV_NB 1  // row batches per wave (gate/up, linear, grouped down)
#endif
#ifndef MOEQ_DOWN1_UB
#define MOEQ_DOWN1_UB 4  // rows per batch (single-token down)
#endif
#ifndef MOEQ_DOWN1_NB
#define MOEQ_DOWN1_NB 2  // row batches per wave (single-token down)
#endif
constexpr int GEMV_UB = MOEQ_GEMV_UB, GEMV_NB = MOEQ_GEMV_NB, DOWN1_UB = MOEQ_DOWN1_UB, DOWN1_NB = MOEQ_DOWN1_NB;

// Launch with hipExtLaunchKernelGGL when timing events are given: the events
// then bracket the kernel's execution itself, not the queue around it.
#define MOEQ_LAUNCH(K, g, b, s, ev, p)                                                \
  do {                                                                                \
    if (ev) hipExtLaunchKernelGGL(K, g, b, 0, s, (ev)->start, (ev)->stop, 0, p);       \
    else hipLaunchKernelGGL(K, g, b, 0, s, p);                                        \
  } while (0)

// IQ2_XXS decodes at several times the ALU cost per byte of the other formats: its
// four rows go in two batches of two, so the first batch's arithmetic overlaps
// the second's transfer; the cheaper formats do better with one batch of four.
#ifndef MOEQ_IQ2_UB
#define MOEQ_IQ2_UB 2  // IQ2_XXS rows per batch
#endif
#ifndef MOEQ_IQ2_NB
#define MOEQ_IQ2_NB 1  // IQ2_XXS row batches per wave
#endif
#ifndef MOEQ_FP8_UB
#define MOEQ_FP8_UB 2  // FP8 block-128 rows per batch (the dense linear at T = 1: 6.27 against 6.74 us with 4)
#endif
#ifndef MOEQ_FP8_NB
#define MOEQ_FP8_NB MOEQ_GEMV_NB  // FP8 block-128 row batches per wave
#endif
template <int FMT> struct GemvRows {
  static constexpr int UB = FMT == FMT_IQ2_XXS ? MOEQ_IQ2_UB : FMT == FMT_FP8_B128 ? MOEQ_FP8_UB : GEMV_UB;
  static constexpr int NB = FMT == FMT_IQ2_XXS ? MOEQ_IQ2_NB : FMT == FMT_FP8_B128 ? MOEQ_FP8_NB : GEMV_NB;
};
// Rows per wave of the GEMV for a format (the host sizes the grid with it).
static int gemv_rows_per_wave(int fmt) {
  switch (fmt) {
    case FMT_IQ2_XXS: return GemvRows<FMT_IQ2_XXS>::UB * GemvRows<FMT_IQ2_XXS>::NB;
    case FMT_FP8_B128: return GemvRows<FMT_FP8_B128>::UB * GemvRows<FMT_FP8_B128>::NB;
    default: return GEMV_UB * GEMV_NB;
  }
}

// Token tile of the wide (several pairs per expert) launches. Every token of the
// tile keeps its activation slices in registers for all of a lane's chunks, so the
// tile shrinks as the chunks per lane grow: gate/up 4 tokens at one chunk per
// lane, 2 at two (K = 4096 in FP4: a 4-token tile spilled about 100 registers and
// an NVFP4 + Q2_K layer at T = 256 took 4.79 ms against 3.06 ms with 2-token
// tiles), 1 at four; down and plain 2 and 4 tokens at one chunk per lane only
// (their wider tiles spill hundreds of registers at two or more).
template <int FMT, int CPL>
static hipError_t gemv_fc(int epi, const GemvParams& p, dim3 g, int mt, hipStream_t s, const LaunchEvents* ev) {
  dim3 b(256);
  constexpr int UB = GemvRows<FMT>::UB, NB = GemvRows<FMT>::NB;
  const bool wide = mt != 1;
  if (epi == EPI_SWIGLU) {
    if (!wide || CPL >= 4) MOEQ_LAUNCH((k_gemv<FMT, CPL, 1, 2, EPI_SWIGLU, ACT_BF16, UB, NB>), g, b, s, ev, p);
    else if (CPL == 2) MOEQ_LAUNCH((k_gemv<FMT, CPL, 2, 2, EPI_SWIGLU, ACT_BF16, UB, NB>), g, b, s, ev, p);
    else MOEQ_LAUNCH((k_gemv<FMT, 1, 4, 2, EPI_SWIGLU, ACT_BF16, UB, NB>), g, b, s, ev, p);
  } else if (epi == EPI_PARTIAL) {
    if (!wide || CPL >= 2) MOEQ_LAUNCH((k_gemv<FMT, CPL, 1, 1, EPI_PARTIAL, ACT_F32, UB, NB>), g, b, s, ev, p);
    else MOEQ_LAUNCH((k_gemv<FMT, 1, 2, 1, EPI_PARTIAL, ACT_F32, UB, NB>), g, b, s, ev, p);
  } else {
    if (!wide || CPL >= 2) MOEQ_LAUNCH((k_gemv<FMT, CPL, 1, 1, EPI_PLAIN, ACT_BF16, UB, NB>), g, b, s, ev, p);
    else MOEQ_LAUNCH((k_gemv<FMT, 1, 4, 1, EPI_PLAIN, ACT_BF16, UB, NB>), g, b, s, ev, p);
  }
  return hipGetLastError();
}

template <int FMT>
static hipError_t gemv_f(int epi, const GemvParams& p, int cpl, dim3 g, int mt, hipStream_t s,
                         const LaunchEvents* ev) {
  switch (cpl) {
    case 1: return gemv_fc<FMT, 1>(epi, p, g, mt, s, ev);
    case 2: return gemv_fc<FMT, 2>(epi, p, g, mt, s, ev);
    case 4: return gemv_fc<FMT, 4>(epi, p, g, mt, s, ev);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(int fmt, int epi, const GemvParams& p, int n_slots, int mt, hipStream_t s,
                       const LaunchEvents* ev) {
  // One token, MXFP4 or NVFP4: the weights go straight into the matrix unit (its
  // scale runs are read 16 bytes at a time, so the scale planes must be 16-byte
  // aligned).
  const bool sc16 = ((uintptr_t)p.w[0].scales % 16 == 0) && ((uintptr_t)p.w[1].scales % 16 == 0) &&
                    p.w[0].sestride % 16 == 0 && p.w[1].sestride % 16 == 0;
  if ((fmt == FMT_MXFP4 || fmt == FMT_NVFP4) && epi == EPI_SWIGLU && p.mode == MODE_DIRECT && mt == 1 && sc16 &&
      gu1_mx4_fits(p.rows, p.cols))
    return launch_gu1_fp4(fmt, p, n_slots, s, ev);
  int lpr, cpl;
  if (!chunk_geometry(fmt, p.cols, &lpr, &cpl)) return hipErrorInvalidValue;
  GemvParams q = p;
  q.lpr = lpr;
  q.chunks = p.cols / weights_per_chunk(fmt);
  int rw_rows = 64 / lpr;
  q.U = gemv_rows_per_wave(fmt);
  q.rows_per_wg = 4 * q.U * rw_rows;
  dim3 g((unsigned)((p.rows + q.rows_per_wg - 1) / q.rows_per_wg), (unsigned)n_slots);
  switch (fmt) {
    case FMT_MXFP4: return gemv_f<FMT_MXFP4>(epi, q, cpl, g, mt, s, ev);
    case FMT_NVFP4: return gemv_f<FMT_NVFP4>(epi, q, cpl, g, mt, s, ev);
    case FMT_Q2_K: return gemv_f<FMT_Q2_K>(epi, q, cpl, g, mt, s, ev);
    case FMT_IQ2_XXS: return gemv_f<FMT_IQ2_XXS>(epi, q, cpl, g, mt, s, ev);
    case FMT_FP8_B128: return gemv_f<FMT_FP8_B128>(epi, q, cpl, g, mt, s, ev);
  }
  return hipErrorInvalidValue;
}

template <int FMT, int MAXW>
static hipError_t down1_fw(const Down1Params& p, int cpl, dim3 g, dim3 b, hipStream_t s) {
  constexpr int UB = DOWN1_UB, NB = DOWN1_NB;
  switch (cpl) {
    case 1: hipLaunchKernelGGL((k_down1<FMT, 1, UB, NB, MAXW>), g, b, 0, s, p); break;
    case 2: hipLaunchKernelGGL((k_down1<FMT, 2, UB, NB, MAXW>), g, b, 0, s, p); break;
    case 4: hipLaunchKernelGGL((k_down1<FMT, 4, UB, NB, MAXW>), g, b, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT>
static hipError_t down1_f(const Down1Params& p, int cpl, dim3 g, dim3 b, hipStream_t s) {
  return p.top_k <= 8 ? down1_fw<FMT, 8>(p, cpl, g, b, s) : down1_fw<FMT, 16>(p, cpl, g, b, s);
}

#ifndef MOEQ_Q2K_MFMA
#define MOEQ_Q2K_MFMA 1
#endif
hipError_t launch_down1(int fmt, const Down1Params& p, hipStream_t s) {
  // MXFP4: straight into the matrix unit (16-byte scale runs and h loads need
  // 16-byte aligned scale planes and h).
  if (fmt == FMT_MXFP4 && down1_mx4_fits(p.rows, p.cols, p.top_k) && (uintptr_t)p.w.scales % 16 == 0 &&
      p.w.sestride % 16 == 0 && (uintptr_t)p.h % 16 == 0)
    return launch_down1_mx4(p, s);
  // Q2_K: the 2-bit codes as FP8 operands of the same instruction (16-byte h loads).
  if (fmt == FMT_Q2_K && MOEQ_Q2K_MFMA && down1_q2k_fits(p.rows, p.cols, p.top_k) && (uintptr_t)p.h % 16 == 0)
    return launch_down1_q2k(p, s);
  int lpr, cpl;
  if (!chunk_geometry(fmt, p.cols, &lpr, &cpl)) return hipErrorInvalidValue;
  Down1Params q = p;
  q.lpr = lpr;
  q.chunks = p.cols / weights_per_chunk(fmt);
  int rw_rows = 64 / lpr;
  q.U = DOWN1_UB * DOWN1_NB;
  if (q.U * rw_rows > 64) q.U = 64 / rw_rows;  // red[] holds 64 rows
  q.rows_per_wg = q.U * rw_rows;
  dim3 g((unsigned)((p.rows + q.rows_per_wg - 1) / q.rows_per_wg)), b((unsigned)(64 * p.top_k));
  switch (fmt) {
    case FMT_MXFP4: return down1_f<FMT_MXFP4>(q, cpl, g, b, s);
    case FMT_NVFP4: return down1_f<FMT_NVFP4>(q, cpl, g, b, s);
    case FMT_Q2_K: return down1_f<FMT_Q2_K>(q, cpl, g, b, s);
    case FMT_IQ2_XXS: return down1_f<FMT_IQ2_XXS>(q, cpl, g, b, s);
    case FMT_FP8_B128: return down1_f<FMT_FP8_B128>(q, cpl, g, b, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moeq
