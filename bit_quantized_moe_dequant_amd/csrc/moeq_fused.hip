// One-launch routed-MoE layer for a single decode token.
//
// A layer at bs=1 streams top_k experts' gate, up and down weights once (80 MB
// for six 2048 x 4096 MXFP4 experts). Two dependent launches each pay the fixed
// cost of a kernel's start-up and drain, which at these sizes is a large share of
// the time, so one launch covers the whole layer:
//
//   1. every work-group issues the loads of its first down item (down weights do
//      not depend on h, only the arithmetic does),
//   2. computes its gate/up items (h = silu(G x) * (U x) rows), statically
//      assigned (items b, b + G, ...),
//   3. publishes its h rows and waits until all G work-groups have,
//   4. computes its down items and the top-k combine.
//
// The grid is the number of work-groups the device holds at once (occupancy
// query), so every work-group is resident and the wait in step 3 ends. h crosses
// work-groups (and XCDs, whose L2s are separate) through agent-scope stores and
// loads, which are coherent without L2 write-back or invalidation. Each wave keeps
// its activation slice (x, then its slot's h) in registers for all its items. The
// last work-group to finish resets the counters for the next launch; a wait that
// runs past a fixed bound sets MOEQ_DEVERR_SPIN and gives up rather than hang.
#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

#ifndef MOEQ_FUSED_GU_ROWS
#define MOEQ_FUSED_GU_ROWS 4
#endif
#ifndef MOEQ_FUSED_DN_ROWS
#define MOEQ_FUSED_DN_ROWS 8
#endif
constexpr int FUSED_GU_ROWS = MOEQ_FUSED_GU_ROWS;  // gate/up rows (of each matrix) per wave per item
constexpr int FUSED_DN_ROWS = MOEQ_FUSED_DN_ROWS;  // down rows per wave (slot) per item

template <int FG, int FD, int CG, int CD>
__global__ __launch_bounds__(512) void k_fused1(FusedParams P) {
  using DG = Dec<FG>;
  using DD = Dec<FD>;
  typedef typename DG::Side SideG;
  typedef typename DD::Side SideD;
  constexpr int XG = XRegs<FG, ACT_BF16>::N, XGS = XRegs<FG, ACT_BF16>::NS;
  constexpr int XD = XRegs<FD, ACT_F32>::N, XDS = XRegs<FD, ACT_F32>::NS;
  constexpr int UG = FUSED_GU_ROWS, UD = FUSED_DN_ROWS;

  __shared__ Iq2Lds lds_g[1];
  __shared__ Iq2Lds lds_d[1];
  __shared__ float red[16][64];
  __shared__ int s_expert[16];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;  // == top_k
  const int G = gridDim.x;
  uint32_t* ctr = P.counters;      // [0] gate/up phases done, [1] exits

  if (threadIdx.x < P.top_k) {
    int e = P.ids[threadIdx.x];
    if (e < 0 || e >= P.n_experts) {
      if (blockIdx.x == 0) atomicOr(P.err, MOEQ_ERRBIT_EXPERT);
      e = -1;
    }
    s_expert[threadIdx.x] = e;
  }
  if constexpr (FG == FMT_IQ2_XXS) iq2_fill_lds(&lds_g[0], P.grid_g, threadIdx.x, blockDim.x);
  if constexpr (FD == FMT_IQ2_XXS) iq2_fill_lds(&lds_d[0], P.grid_d, threadIdx.x, blockDim.x);
  __syncthreads();

  const int lg = P.lpr_g, rwg = 64 / lg, lrg = lane & (lg - 1), rsg = lane / lg;
  const int ld = P.lpr_d, rwd = 64 / ld, lrd = lane & (ld - 1), rsd = lane / ld;
  const int rows_gu_item = nw * UG * rwg;  // flattened (slot, row) pairs per gate/up item
  const int rows_dn_item = UD * rwd;       // output rows per down item

  // Down weights of this work-group's first down item: issued before any
  // gate/up work so their HBM traffic overlaps the gate/up phase.
  const int e_dn = s_expert[wave];
  WView WD;
  WD.data = P.d.data + (size_t)(e_dn < 0 ? 0 : e_dn) * P.d.estride;
  WD.scales = P.d.scales + (size_t)(e_dn < 0 ? 0 : e_dn) * P.d.sestride;
  WD.rows = P.hidden;
  WD.cols = P.inter;
  u32x4 qd[UD][CD];
  SideD sdd[UD][CD];
  auto load_dn = [&](int item) {
    const int r0 = item * rows_dn_item;
#pragma unroll
    for (int u = 0; u < UD; u++) {
      const int r = r0 + u * rwd + rsd;
#pragma unroll
      for (int c = 0; c < CD; c++) {
        if (item < P.n_dn && e_dn >= 0 && r < P.hidden && lrd + ld * c < P.chunks_d) {
          qd[u][c] = ld16(DD::chunk_ptr(WD, r, lrd + ld * c));
          sdd[u][c] = DD::side(WD, r, lrd + ld * c);
        } else {
          qd[u][c] = u32x4{0u, 0u, 0u, 0u};
          sdd[u][c] = SideD{};
        }
      }
    }
  };
  load_dn(blockIdx.x);

  // x slice (same token for every slot)
  uint32_t xg[CG][XG];
  float xgs[CG][XGS];
#pragma unroll
  for (int c = 0; c < CG; c++) {
    if (lrg + lg * c < P.chunks_g) {
      DG::template load_x<ACT_BF16>(P.x, lrg + lg * c, xg[c], xgs[c]);
    } else {
#pragma unroll
      for (int j = 0; j < XG; j++) xg[c][j] = 0u;
#pragma unroll
      for (int j = 0; j < XGS; j++) xgs[c][j] = 0.f;
    }
  }

  // ---------------- gate/up items blockIdx.x, blockIdx.x + G, ...
  for (int t = blockIdx.x; t < P.n_gu; t += G) {
    const int pr0 = t * rows_gu_item + wave * UG * rwg;  // first flattened pair-row of this wave
    const int slot = pr0 / P.inter;
    const int e = slot < P.top_k ? s_expert[slot] : -1;
    u32x4 q[2][UG][CG];
    SideG sd[2][UG][CG];
    WView W[2];
#pragma unroll
    for (int m = 0; m < 2; m++) {
      W[m].data = P.g[m].data + (size_t)(e < 0 ? 0 : e) * P.g[m].estride;
      W[m].scales = P.g[m].scales + (size_t)(e < 0 ? 0 : e) * P.g[m].sestride;
      W[m].rows = P.inter;
      W[m].cols = P.hidden;
    }
#pragma unroll
    for (int m = 0; m < 2; m++)
#pragma unroll
      for (int u = 0; u < UG; u++) {
        const int pr = pr0 + u * rwg + rsg;
        const int r = pr - slot * P.inter;
#pragma unroll
        for (int c = 0; c < CG; c++) {
          if (e >= 0 && pr < P.top_k * P.inter && r < P.inter && lrg + lg * c < P.chunks_g) {
            q[m][u][c] = ld16(DG::chunk_ptr(W[m], r, lrg + lg * c));
            sd[m][u][c] = DG::side(W[m], r, lrg + lg * c);
          } else {
            q[m][u][c] = u32x4{0u, 0u, 0u, 0u};
            sd[m][u][c] = SideG{};
          }
        }
      }
    float acc[2][UG];
#pragma unroll
    for (int m = 0; m < 2; m++)
#pragma unroll
      for (int u = 0; u < UG; u++) {
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < CG; c++) a = DG::template dot<ACT_BF16>(q[m][u][c], sd[m][u][c], xg[c], xgs[c], a, &lds_g[0]);
        acc[m][u] = a;
      }
    group_reduce<UG>(acc[0], lg, lane);
    group_reduce<UG>(acc[1], lg, lane);
    const int nf = UG >= lg ? UG / lg : 1;
    const bool writer = UG >= lg ? true : ((lrg % (lg / UG)) == 0);
    const int vi0 = (lrg * UG) / lg;
    if (writer) {
      const float s2g = (FG == FMT_NVFP4 && e >= 0) ? P.g[0].scale2[e] : 1.0f;
      const float s2u = (FG == FMT_NVFP4 && e >= 0) ? P.g[1].scale2[e] : 1.0f;
#pragma unroll
      for (int i = 0; i < UG; i++) {
        if (i < nf) {
          const int pr = pr0 + (vi0 + i) * rwg + rsg;
          if (pr < P.top_k * P.inter && slot < P.top_k) {
            const int r = pr - slot * P.inter;
            // agent-scope store: coherent across the XCDs' L2s, no write-back needed
            if (r < P.inter)
              __hip_atomic_store(&P.h[(size_t)slot * P.inter + r],
                                 e >= 0 ? silu_mul(acc[0][i] * s2g, acc[1][i] * s2u) : 0.f, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
  }

  // ---------------- publish this work-group's h rows, then wait for everyone's
  __builtin_amdgcn_s_waitcnt(0);  // this wave's h stores are acknowledged
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(&ctr[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0;
    while (__hip_atomic_load(&ctr[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)G) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > P.spin_limit) {
        atomicOr(P.err, MOEQ_ERRBIT_SPIN);
        break;
      }
    }
  }
  __syncthreads();

  // h slice of this wave's slot, read with agent-scope loads (never a stale L2 copy)
  uint32_t xd[CD][XD];
  float xds[CD][XDS];
  const float* hrow = P.h + (size_t)wave * P.inter;
#pragma unroll
  for (int c = 0; c < CD; c++) {
    if (lrd + ld * c < P.chunks_d) {
      DD::template load_x<ACT_F32_COHERENT>(hrow, lrd + ld * c, xd[c], xds[c]);
    } else {
#pragma unroll
      for (int j = 0; j < XD; j++) xd[c][j] = 0u;
#pragma unroll
      for (int j = 0; j < XDS; j++) xds[c][j] = 0.f;
    }
  }
  const float wk = e_dn >= 0 ? P.rw[wave] * ((FD == FMT_NVFP4) ? P.d.scale2[e_dn] : 1.0f) : 0.f;

  // ---------------- down items blockIdx.x, blockIdx.x + G, ...
  for (int t = blockIdx.x; t < P.n_dn; t += G) {
    if (t != (int)blockIdx.x) load_dn(t);
    float acc[UD];
#pragma unroll
    for (int u = 0; u < UD; u++) {
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < CD; c++) a = DD::template dot<ACT_F32>(qd[u][c], sdd[u][c], xd[c], xds[c], a, &lds_d[0]);
      acc[u] = a;
    }
    group_reduce<UD>(acc, ld, lane);
    const int nf = UD >= ld ? UD / ld : 1;
    const bool writer = UD >= ld ? true : ((lrd % (ld / UD)) == 0);
    const int vi0 = (lrd * UD) / ld;
    if (writer) {
#pragma unroll
      for (int i = 0; i < UD; i++) {
        if (i < nf) red[wave][(vi0 + i) * rwd + rsd] = e_dn >= 0 ? acc[i] * wk : 0.f;
      }
    }
    __syncthreads();
    const int r0 = t * rows_dn_item;
    for (int i = threadIdx.x; i < rows_dn_item; i += blockDim.x) {
      const int r = r0 + i;
      if (r < P.hidden) {
        float y = 0.f;
        for (int k = 0; k < nw; k++) y += red[k][i];
        P.y[r] = y;
      }
    }
    __syncthreads();
  }

  // the last work-group out resets the counters for the next launch
  if (threadIdx.x == 0) {
    uint32_t done = __hip_atomic_fetch_add(&ctr[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (uint32_t)G - 1) {
      __hip_atomic_store(&ctr[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ctr[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Instantiated pairs (gate/up format, down format) with chunks-per-lane (1 or 2
// for gate/up, 1 for down); other geometries use the two-launch path.
template <int FG, int FD>
static hipError_t fused_fd(const FusedParams& p, int cg, dim3 g, dim3 b, hipStream_t s) {
  if (cg == 1) hipLaunchKernelGGL((k_fused1<FG, FD, 1, 1>), g, b, 0, s, p);
  else hipLaunchKernelGGL((k_fused1<FG, FD, 2, 1>), g, b, 0, s, p);
  return hipGetLastError();
}

bool fused1_supported(int fg, int fd, int hidden, int inter, int top_k) {
  int lg, cg, ld, cd;
  if (!chunk_geometry(fg, hidden, &lg, &cg) || !chunk_geometry(fd, inter, &ld, &cd)) return false;
  if (cg > 2 || cd != 1 || top_k > 8) return false;
  if (inter % (FUSED_GU_ROWS * (64 / lg))) return false;  // a wave's gate/up rows stay in one slot
  if (FUSED_DN_ROWS * (64 / ld) > 64) return false;  // red[] rows
  const bool pair_ok = (fg == fd) || (fg == FMT_NVFP4 && fd == FMT_Q2_K) || (fg == FMT_IQ2_XXS && fd == FMT_Q2_K);
  return pair_ok;
}

#ifndef MOEQ_FUSED_GRID
#define MOEQ_FUSED_GRID 1024  // upper bound; the occupancy query sets the grid
#endif

// Work-groups of this kernel the current device holds at once. Queried once per
// (device, kernel, block size) and kept: it is a property of the device.
template <int FG, int FD, int CG>
static int fused_capacity(int threads) {
  static int cached[64][17];  // [device][top_k]
  int dev_id = 0;
  if (hipGetDevice(&dev_id) != hipSuccess || dev_id < 0 || dev_id >= 64) return 0;
  int& slot = cached[dev_id][threads / 64];
  if (slot > 0) return slot;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_fused1<FG, FD, CG, 1>, threads, 0) !=
      hipSuccess)
    return 0;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  slot = per_cu * cus;
  return slot;
}

hipError_t launch_fused1(int fg, int fd, const FusedParams& p0, hipStream_t s) {
  FusedParams p = p0;
  int cg, cd;
  chunk_geometry(fg, p.hidden, &p.lpr_g, &cg);
  chunk_geometry(fd, p.inter, &p.lpr_d, &cd);
  p.chunks_g = p.hidden / weights_per_chunk(fg);
  p.chunks_d = p.inter / weights_per_chunk(fd);
  const int rows_gu_item = p.top_k * FUSED_GU_ROWS * (64 / p.lpr_g);
  const int rows_dn_item = FUSED_DN_ROWS * (64 / p.lpr_d);
  p.n_gu = (p.top_k * p.inter + rows_gu_item - 1) / rows_gu_item;
  p.n_dn = (p.hidden + rows_dn_item - 1) / rows_dn_item;
  if (p.spin_limit == 0) p.spin_limit = 1u << 24;
  const int threads = 64 * p.top_k;
  int cap = 0;
#define MOEQ_FD(A, B)                                                             \
  if (fg == A && fd == B) cap = cg == 1 ? fused_capacity<A, B, 1>(threads) : fused_capacity<A, B, 2>(threads);
  MOEQ_FD(FMT_MXFP4, FMT_MXFP4)
  MOEQ_FD(FMT_NVFP4, FMT_NVFP4)
  MOEQ_FD(FMT_Q2_K, FMT_Q2_K)
  MOEQ_FD(FMT_IQ2_XXS, FMT_IQ2_XXS)
  MOEQ_FD(FMT_FP8_B128, FMT_FP8_B128)
  MOEQ_FD(FMT_NVFP4, FMT_Q2_K)
  MOEQ_FD(FMT_IQ2_XXS, FMT_Q2_K)
#undef MOEQ_FD
  if (cap <= 0) return hipErrorInvalidValue;
  int grid = cap < MOEQ_FUSED_GRID ? cap : MOEQ_FUSED_GRID;
  if (grid > p.n_dn) grid = p.n_dn;  // every work-group owns at least one down item
  dim3 g((unsigned)grid), b((unsigned)threads);
#define MOEQ_FD(A, B) \
  if (fg == A && fd == B) return fused_fd<A, B>(p, cg, g, b, s);
  MOEQ_FD(FMT_MXFP4, FMT_MXFP4)
  MOEQ_FD(FMT_NVFP4, FMT_NVFP4)
  MOEQ_FD(FMT_Q2_K, FMT_Q2_K)
  MOEQ_FD(FMT_IQ2_XXS, FMT_IQ2_XXS)
  MOEQ_FD(FMT_FP8_B128, FMT_FP8_B128)
  MOEQ_FD(FMT_NVFP4, FMT_Q2_K)
  MOEQ_FD(FMT_IQ2_XXS, FMT_Q2_K)
#undef MOEQ_FD
  return hipErrorInvalidValue;
}

}  // namespace moeq
