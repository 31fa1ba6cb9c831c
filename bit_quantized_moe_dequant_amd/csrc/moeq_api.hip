// C ABI of the library: argument checks, workspace layout and kernel dispatch.
// Everything here runs on the host; kernels are launched asynchronously on the
// caller's stream and nothing is allocated or synchronised on the forward path.
#include <string.h>
#include <math.h>

#include "moeq.h"
#include "moeq_kernels.h"

#include <cmath>
#include <mutex>

using namespace moeq;

namespace {

constexpr int PREFILL_MIN_T = 128;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int block_k(int fmt) {
  switch (fmt) {
    case MOEQ_FMT_MXFP4: return 32;
    case MOEQ_FMT_NVFP4: return 16;
    case MOEQ_FMT_Q2_K: return 256;
    case MOEQ_FMT_IQ2_XXS: return 256;
    case MOEQ_FMT_FP8_B128: return 128;
    case MOEQ_FMT_MXFP8: return 32;
    case MOEQ_FMT_FP8_B32: return 32;
    case MOEQ_FMT_MXFP8_TILED: return 512;
  }
  return 0;
}

// Formats for dense linears only (moeq_linear, moeq_dequant), not for layers.
bool dense_only(int fmt) { return fmt == MOEQ_FMT_MXFP8 || fmt == MOEQ_FMT_FP8_B32 || fmt == MOEQ_FMT_MXFP8_TILED; }

size_t plane_bytes(int fmt, int rows, int cols, int plane) {
  int bk = block_k(fmt);
  if (bk == 0 || rows <= 0 || cols <= 0 || cols % bk || (plane != 0 && plane != 1)) return 0;
  size_t n = (size_t)rows * cols;
  switch (fmt) {
    case MOEQ_FMT_MXFP4: return plane == 0 ? n / 2 : n / 32;
    case MOEQ_FMT_NVFP4: return plane == 0 ? n / 2 : n / 16;
    case MOEQ_FMT_Q2_K: return (size_t)rows * (cols / 256) * (plane == 0 ? 64 : 20);
    case MOEQ_FMT_IQ2_XXS: return (size_t)rows * (cols / 256) * (plane == 0 ? 64 : 2);
    case MOEQ_FMT_FP8_B128:
      if (rows % 128) return 0;
      return plane == 0 ? n : (size_t)(rows / 128) * (cols / 128);
    case MOEQ_FMT_FP8_B32:
      if (rows % 32) return 0;
      return plane == 0 ? n : (size_t)(rows / 32) * (cols / 32);
    case MOEQ_FMT_MXFP8: return plane == 0 ? n : n / 32;
    case MOEQ_FMT_MXFP8_TILED:
      if (rows % 16) return 0;
      return plane == 0 ? n : n / 32;
  }
  return 0;
}

WeightRef ref_of(const moeq_weight& w) {
  WeightRef r;
  r.data = (const uint8_t*)w.data;
  r.scales = (const uint8_t*)w.scales;
  r.estride = w.expert_stride;
  r.sestride = w.scale_expert_stride;
  r.scale2 = w.fmt == MOEQ_FMT_NVFP4 ? w.scale2 : nullptr;
  return r;
}

// Checks a weight descriptor; gemv = the tensor is used by the GEMV kernels.
int check_weight(const moeq_weight* w, bool gemv) {
  if (!w) return MOEQ_E_INVAL;
  if (block_k(w->fmt) == 0) return MOEQ_E_FMT;
  if (w->n_experts <= 0) return MOEQ_E_INVAL;
  size_t p0 = plane_bytes(w->fmt, w->rows, w->cols, 0), p1 = plane_bytes(w->fmt, w->rows, w->cols, 1);
  if (p0 == 0 || p1 == 0) return MOEQ_E_SHAPE;
  if (w->cols % weights_per_chunk(w->fmt)) return MOEQ_E_SHAPE;
  if (gemv) {
    int lpr, cpl;
    if (!chunk_geometry(w->fmt, w->cols, &lpr, &cpl)) return MOEQ_E_SHAPE;
  }
  if (!w->data || !w->scales) return MOEQ_E_INVAL;
  if (!aligned(w->data, 16) || !aligned(w->scales, 4)) return MOEQ_E_ALIGN;
  if (w->n_experts > 1) {
    if (w->expert_stride < p0 || w->scale_expert_stride < p1) return MOEQ_E_INVAL;
    if (w->expert_stride % 16 || w->scale_expert_stride % 4) return MOEQ_E_ALIGN;
  }
  if (w->fmt == MOEQ_FMT_NVFP4 && (!w->scale2 || !aligned(w->scale2, 4))) return MOEQ_E_INVAL;
  if (w->fmt == MOEQ_FMT_IQ2_XXS && !w->grid) return MOEQ_E_INVAL;
  return MOEQ_OK;
}

int check_layer(const moeq_layer* L) {
  if (!L) return MOEQ_E_INVAL;
  if (L->hidden <= 0 || L->inter <= 0 || L->n_experts <= 0 || L->top_k < 1 || L->top_k > 16) return MOEQ_E_INVAL;
  if (L->n_experts > 1024) return MOEQ_E_SHAPE;
  int rc;
  if ((rc = check_weight(&L->gate, true)) || (rc = check_weight(&L->up, true)) || (rc = check_weight(&L->down, true)))
    return rc;
  if (L->gate.rows != L->inter || L->gate.cols != L->hidden) return MOEQ_E_SHAPE;
  if (L->up.rows != L->inter || L->up.cols != L->hidden) return MOEQ_E_SHAPE;
  if (L->down.rows != L->hidden || L->down.cols != L->inter) return MOEQ_E_SHAPE;
  if (L->gate.fmt != L->up.fmt) return MOEQ_E_FMT;
  if (dense_only(L->gate.fmt) || dense_only(L->down.fmt)) return MOEQ_E_FMT;
  if (L->gate.n_experts < L->n_experts || L->up.n_experts < L->n_experts || L->down.n_experts < L->n_experts)
    return MOEQ_E_INVAL;
  // h is read as fp32 in 16-byte pieces; x as bf16 in 16-byte pieces
  if (L->inter % 4 || L->hidden % 8) return MOEQ_E_SHAPE;
  return MOEQ_OK;
}

// From PREFILL_MIN_T tokens each MXFP4 projection (gate/up, down) takes the W4A8
// grouped GEMM, whatever the format of the other one (a mixed IQ2_XXS / MXFP4
// layer, DeepSeekv4 Flash for 1x Spark forum thread, second post: one grouped
// GEMM per projection).
bool prefill_buffers(const moeq_layer* L, int T) {
  return T >= PREFILL_MIN_T && (L->gate.fmt == MOEQ_FMT_MXFP4 || L->down.fmt == MOEQ_FMT_MXFP4);
}

struct WsLayout {
  size_t route, h, partial, xq, xs, hq, hs, dq, ds, total;
  int P;
  uint32_t* err;  // device error word the kernels OR into (null: the workspace's own)
};

WsLayout ws_layout(const moeq_layer* L, int T) {
  const size_t P = (size_t)T * L->top_k;
  WsLayout w;
  w.P = (int)P;
  size_t off = 256;  // header: device error word at 0
  w.route = off;
  off += align_up(RouteView::words(L->n_experts, (int)P) * 4, 256);
  w.h = off;
  off += align_up(P * L->inter * 4, 256);
  w.partial = off;
  off += T > 1 ? align_up(P * L->hidden * 4, 256) : 0;
  w.xq = w.xs = w.hq = w.hs = w.dq = w.ds = 0;
  w.err = nullptr;
  if (T > 1 && L->down.fmt == MOEQ_FMT_Q2_K && dn_q2k_g_fits(L->hidden, L->inter)) {
    // digit planes of h for the grouped Q2_K down
    w.dq = off;
    off += align_up(dn_q2k_g_digit_bytes((long)P, L->inter), 256);
    w.ds = off;
    off += align_up(dn_q2k_g_scale_bytes((long)P, L->inter), 256);
  }
  if (prefill_buffers(L, T)) {
    w.xq = off;
    off += align_up((size_t)T * L->hidden, 256);
    w.xs = off;
    off += align_up((size_t)T * L->hidden / 32, 256);
    w.hq = off;
    off += align_up(P * L->inter, 256);
    w.hs = off;
    off += align_up(P * L->inter / 32, 256);
  }
  w.total = off;
  return w;
}

int check_ws(const moeq_layer* L, int T, void* ws, size_t ws_bytes) {
  if (!ws) return MOEQ_E_WORKSPACE;
  if (!aligned(ws, 256)) return MOEQ_E_ALIGN;
  if (ws_bytes < ws_layout(L, T).total) return MOEQ_E_WORKSPACE;
  return MOEQ_OK;
}

inline int hip_rc(hipError_t e) { return e == hipSuccess ? MOEQ_OK : MOEQ_E_HIP; }
inline hipStream_t S(void* s) { return (hipStream_t)s; }
inline uint32_t* err_word(void* ws) { return (uint32_t*)ws; }
inline uint32_t* err_of(void* ws, const WsLayout& lay) { return lay.err ? lay.err : err_word(ws); }
inline RouteView route_view(const moeq_layer* L, void* ws, const WsLayout& lay) {
  RouteView rv;
  rv.base = (int32_t*)((uint8_t*)ws + lay.route);
  rv.E = L->n_experts;
  rv.P = lay.P;
  return rv;
}

GemvParams gemv_params(const moeq_layer* L, const moeq_weight& a, const moeq_weight* b, void* ws,
                       const WsLayout& lay) {
  GemvParams p;
  memset(&p, 0, sizeof(p));
  p.w[0] = ref_of(a);
  p.w[1] = b ? ref_of(*b) : ref_of(a);
  p.grid = a.grid;
  p.rows = a.rows;
  p.cols = a.cols;
  p.n_experts = L ? L->n_experts : a.n_experts;
  p.top_k = L ? L->top_k : 1;
  if (ws) {
    p.route = route_view(L, ws, lay);
    p.err = err_of(ws, lay);
  }
  return p;
}

// Token tile of the grouped GEMVs (T > 1): the pairs of an expert are processed
// this many at a time. The tile's register cost (activations of every token it
// holds) lowers occupancy, and at a few tokens per expert most of it would be
// padding, so the width follows the expected pairs per touched expert under
// uniform routing, P / (E (1 - (1 - K/E)^T)). #ifndef lets a build pin it.
#ifndef MOEQ_GROUPED_WIDE_FROM
#define MOEQ_GROUPED_WIDE_FROM 2.5
#endif
double pairs_per_expert(const moeq_layer* L, int T) {
  const double E = L->n_experts, K = L->top_k;
  const double touched = E * (1.0 - std::pow(1.0 - K / E, (double)T));
  return (double)T * K / (touched > 1.0 ? touched : 1.0);
}
bool grouped_wide(const moeq_layer* L, int T) { return pairs_per_expert(L, T) >= MOEQ_GROUPED_WIDE_FROM; }

// IQ2_XXS gate/up for T > 1: the wide kernel (up to four 16-token tiles per decode)
// from this many pairs per expert (T K / E), the one-tile kernel below it.
// IQ2_XXS + Q2_K at T = 512 / 768 / 1024 / 1536 / 2048 (12 / 18 / 24 / 36 / 48
// pairs): 1257 / 1768 / 2238 / 3230 / 4201 us with the one-tile kernel against
// 1687 / 2004 / 2293 / 2877 / 3503 us with the wide one.
#ifndef MOEQ_IQ2_WIDE_FROM
#define MOEQ_IQ2_WIDE_FROM 28.0
#endif

// Q2_K down at T > 1 off the direct path: partials on the block-scaled FP8
// instruction (each expert's weights read once, h's digits made once per pair)
// below MOEQ_Q2K_G_BELOW pairs per touched expert, else on the bf16 instruction
// (decode once per 16 tokens) from MOEQ_DN_Q2K_FROM pairs. The FP8 kernel was
// faster at every load measured: IQ2_XXS + Q2_K layers at T = 64 / 256 / 2048 (2,
// 6 and 48 pairs) took 782 / 1201 / 3448 us against 1108 (direct) / 1423 / 3768 us
// (bf16). The bf16 kernel stays for intermediate sizes above 2048.
#ifndef MOEQ_DN_Q2K_FROM
#define MOEQ_DN_Q2K_FROM 2.5
#endif
#ifndef MOEQ_Q2K_G_BELOW
#define MOEQ_Q2K_G_BELOW 1e30
#endif

// MXFP4 decode at T > 1 on the block-scaled matrix instruction (1), or as GEMVs (0).
#ifndef MOEQ_MX4_BATCHED
#define MOEQ_MX4_BATCHED 1
#endif
// NVFP4 gate/up off the direct path: on the same token-grouped kernel (one pair per
// instruction) from this many pairs per touched expert, as grouped GEMVs below it.
// Since the grouped kernel fits three work-groups per CU it is ahead at every load
// (NVFP4 + Q2_K at T = 24 / 32: 266 / 327 us against 317 / 397 us with the GEMVs),
// so the GEMVs no longer take this path.
#ifndef MOEQ_NV4_GROUPED_FROM
#define MOEQ_NV4_GROUPED_FROM 0.0
#endif

// Scale plane read in 16-byte runs by the matrix-instruction kernels.
bool scales16(const moeq_weight& w) {
  return aligned(w.scales, 16) && (w.n_experts == 1 || w.scale_expert_stride % 16 == 0);
}

// Decode of a few tokens without grouping: the single-token kernels run over every
// (token, slot) pair directly, with no routing, no partials and no combine (an
// expert routed by several tokens is read once per pair). The gate/up takes this
// path for MXFP4 up to MOEQ_FP4_DIRECT_MAX_T tokens and for NVFP4 up to
// MOEQ_NV4_DIRECT_MAX_T (the block-scaled matrix-unit kernels; NVFP4 + Q2_K at
// T = 8 / 12 / 16: 122 / 170 / 217 us direct against 118 / 159 / 197 us grouped); the down for MXFP4 up to MOEQ_FP4_DIRECT_MAX_T, for Q2_K below a load
// of MOEQ_Q2K_DIRECT_BELOW pairs per touched expert (0 turns that off; NVFP4 + Q2_K
// at T = 2 / 4 / 8 / 16 / 64: 46.3 / 87.3 / 160.0 / 294.6 / 1024 us direct against
// 58.4 / 89.3 / 149.8 / 255.3 / 702 us with the grouped FP8 down). The routing kernel
// runs only when a projection takes the grouped path.
// (MXFP4 layer at T = 8 / 12 / 16 / 24 / 32: 107.7 / 155.5 / 203 / 299 / 397 us
// direct against 111 / 151.5 / 188 / 252.5 / 309.6 us grouped, with the grouped
// kernels' two-pair tiles and row-split down.)
#ifndef MOEQ_FP4_DIRECT_MAX_T
#define MOEQ_FP4_DIRECT_MAX_T 8
#endif
#ifndef MOEQ_NV4_DIRECT_MAX_T
#define MOEQ_NV4_DIRECT_MAX_T 4
#endif
// IQ2_XXS gate/up: the dequantize + GEMV over every pair below this load (pairs per
// touched expert), i.e. up to 3 tokens over 256 experts: IQ2_XXS + Q2_K at T = 2 /
// 3 / 4 / 8 / 16 / 32 took 41.7 / 58.0 / 75.1 / 143.5 / 259 / 479 us with the GEMV
// against 49.2 / 65.3 / 73.0 / 126.5 / 210 / 333 us with the token-grouped kernel.
#ifndef MOEQ_IQ2_DIRECT_BELOW
#define MOEQ_IQ2_DIRECT_BELOW 1.03
#endif
#ifndef MOEQ_Q2K_DIRECT_BELOW
#define MOEQ_Q2K_DIRECT_BELOW 1.06
#endif
bool gu_direct(const moeq_layer* L, int T) {
  if (T == 1) return true;
  if (L->gate.fmt == MOEQ_FMT_IQ2_XXS)  // the dequantize + GEMV over every pair
    return T >= 1 && L->up.fmt == MOEQ_FMT_IQ2_XXS && pairs_per_expert(L, T) < MOEQ_IQ2_DIRECT_BELOW;
  const int max_t = L->gate.fmt == MOEQ_FMT_MXFP4 ? MOEQ_FP4_DIRECT_MAX_T
                    : L->gate.fmt == MOEQ_FMT_NVFP4 ? MOEQ_NV4_DIRECT_MAX_T
                                                    : 0;
  return T >= 1 && T <= max_t && L->gate.fmt == L->up.fmt && gu1_mx4_fits(L->inter, L->hidden) &&
         scales16(L->gate) && scales16(L->up);
}
bool dn_direct(const moeq_layer* L, int T, const float* h) {
  if (T == 1) return true;
  if (T < 1 || !aligned(h, 16)) return false;
  if (L->down.fmt == MOEQ_FMT_MXFP4)
    return T <= MOEQ_FP4_DIRECT_MAX_T && down1_mx4_fits(L->hidden, L->inter, L->top_k) && scales16(L->down);
  if (L->down.fmt == MOEQ_FMT_Q2_K)
    return pairs_per_expert(L, T) < MOEQ_Q2K_DIRECT_BELOW && down1_q2k_fits(L->hidden, L->inter, L->top_k);
  return false;
}

int run_gate_up(const moeq_layer* L, const void* x, const int32_t* ids, int T, float* h, void* ws, const WsLayout& lay,
                hipStream_t s, const LaunchEvents* ev = nullptr) {
  GemvParams p = gemv_params(L, L->gate, &L->up, ws, lay);
  p.act = x;
  p.ids = ids;
  p.T = T;
  p.out = h;
  if (gu_direct(L, T)) {
    p.mode = MODE_DIRECT;
    return hip_rc(launch_gemv(L->gate.fmt, EPI_SWIGLU, p, T * L->top_k, 1, s, ev));
  }
  p.mode = MODE_GROUPED;
  int slots = L->n_experts + 1;
  if (T * L->top_k + 1 < slots) slots = T * L->top_k + 1;
  if (L->gate.fmt == MOEQ_FMT_IQ2_XXS && gu_iq2_fits(L->inter, L->hidden))
    return hip_rc(launch_gu_iq2(p, slots, (double)T * L->top_k >= MOEQ_IQ2_WIDE_FROM * L->n_experts, s));
  const bool fp4_g = (MOEQ_MX4_BATCHED && L->gate.fmt == MOEQ_FMT_MXFP4) ||
                     (L->gate.fmt == MOEQ_FMT_NVFP4 && pairs_per_expert(L, T) >= MOEQ_NV4_GROUPED_FROM);
  if (fp4_g && gu_mx4_g_fits(L->inter, L->hidden) && scales16(L->gate) && scales16(L->up))
    return hip_rc(launch_gu_fp4_g(L->gate.fmt, p, slots, s));
  return hip_rc(launch_gemv(L->gate.fmt, EPI_SWIGLU, p, slots, grouped_wide(L, T) ? 4 : 1, s, ev));
}

int run_down(const moeq_layer* L, const float* h, const int32_t* ids, const float* rw, int T, float* y, void* ws,
             const WsLayout& lay, hipStream_t s) {
  if (dn_direct(L, T, h)) {
    Down1Params d;
    memset(&d, 0, sizeof(d));
    d.T = T;
    d.w = ref_of(L->down);
    d.grid = L->down.grid;
    d.rows = L->down.rows;
    d.cols = L->down.cols;
    d.n_experts = L->n_experts;
    d.top_k = L->top_k;
    d.h = h;
    d.ids = ids;
    d.rw = rw;
    d.y = y;
    d.err = err_of(ws, lay);
    return hip_rc(launch_down1(L->down.fmt, d, s));
  }
  GemvParams p = gemv_params(L, L->down, nullptr, ws, lay);
  p.act = h;
  p.ids = ids;
  p.rw = rw;
  p.T = T;
  p.mode = MODE_GROUPED;
  float* partial = (float*)((uint8_t*)ws + lay.partial);
  p.out = partial;
  int slots = L->n_experts + 1;
  if (T * L->top_k + 1 < slots) slots = T * L->top_k + 1;
  int rc;
  const double ppe = pairs_per_expert(L, T);
  if (L->down.fmt == MOEQ_FMT_Q2_K && ppe < MOEQ_Q2K_G_BELOW && lay.dq && aligned(h, 16))
    rc = hip_rc(launch_dn_q2k_g(p, slots, (uint8_t*)ws + lay.dq, (uint8_t*)ws + lay.ds, s));
  else if (L->down.fmt == MOEQ_FMT_Q2_K && ppe >= MOEQ_DN_Q2K_FROM &&
           dn_q2k_fits(L->hidden, L->inter, (long)T * L->top_k))
    rc = hip_rc(launch_dn_q2k(p, slots, s));
  else if (L->down.fmt == MOEQ_FMT_IQ2_XXS && pairs_per_expert(L, T) >= MOEQ_DN_Q2K_FROM &&
           dn_q2k_fits(L->hidden, L->inter, (long)T * L->top_k))
    rc = hip_rc(launch_dn_iq2(p, slots, s));
  else if (MOEQ_MX4_BATCHED && L->down.fmt == MOEQ_FMT_MXFP4 && dn_mx4_g_fits(L->hidden, L->inter) &&
           scales16(L->down))
    rc = hip_rc(launch_dn_mx4_g(p, slots, s));
  else
    rc = hip_rc(launch_gemv(L->down.fmt, EPI_PARTIAL, p, slots, grouped_wide(L, T) ? 2 : 1, s));
  if (rc) return rc;
  return hip_rc(launch_combine(partial, T, L->top_k, L->hidden, y, s));
}

// The W4A8 prefill stage of the gate/up pair (gate_up) or of down: its weights
// MXFP4, K advancing in chunks of 256 (hidden and inter multiples of 256), scale
// planes staged in 8-byte pieces.
int check_prefill(const moeq_layer* L, bool gate_up) {
  if (gate_up ? (L->gate.fmt != MOEQ_FMT_MXFP4 || L->up.fmt != MOEQ_FMT_MXFP4) : L->down.fmt != MOEQ_FMT_MXFP4)
    return MOEQ_E_FMT;
  if (L->hidden % 256 || L->inter % 256) return MOEQ_E_SHAPE;
  if (gate_up) {
    for (const moeq_weight* w : {&L->gate, &L->up})
      if (!aligned(w->scales, 8) || w->scale_expert_stride % 8) return MOEQ_E_ALIGN;
  } else if (!aligned(L->down.scales, 8) || L->down.scale_expert_stride % 8) {
    return MOEQ_E_ALIGN;
  }
  return MOEQ_OK;
}

// The prefill kernels address A (MXFP8 x, then MXFP8 h) with 32-bit offsets.
bool prefill_a_fits(const moeq_layer* L, int T) {
  const size_t lim = (size_t)1 << 31;
  return (size_t)T * L->hidden < lim && (size_t)T * L->top_k * L->inter < lim;
}

int run_prefill_gate_up(const moeq_layer* L, const uint8_t* xq, const uint8_t* xs, int T, float* h_f32,
                               uint8_t* hq, uint8_t* hs, void* ws, const WsLayout& lay, hipStream_t s) {
  if (!prefill_a_fits(L, T)) return MOEQ_E_SHAPE;
  PrefillParams p;
  memset(&p, 0, sizeof(p));
  p.w[0] = ref_of(L->gate);
  p.w[1] = ref_of(L->up);
  p.rows = L->inter;
  p.cols = L->hidden;
  p.n_experts = L->n_experts;
  p.top_k = L->top_k;
  p.aq = xq;
  p.as = xs;
  p.route = route_view(L, ws, lay);
  p.h_f32 = h_f32;
  p.hq = hq;
  p.hs = hs;
  int slots = L->n_experts + 1;
  if (T * L->top_k + 1 < slots) slots = T * L->top_k + 1;
  return hip_rc(launch_prefill(true, p, slots, s));
}

int run_prefill_down(const moeq_layer* L, const uint8_t* hq, const uint8_t* hs, const float* rw, int T, float* y,
                            void* ws, const WsLayout& lay, hipStream_t s) {
  if (!prefill_a_fits(L, T)) return MOEQ_E_SHAPE;
  PrefillParams p;
  memset(&p, 0, sizeof(p));
  p.w[0] = ref_of(L->down);
  p.w[1] = p.w[0];
  // the kernel's second weight tile of each wave: the same matrix 128 rows on
  p.w[1].data += (size_t)128 * (L->inter / 2);
  p.w[1].scales += (size_t)128 * (L->inter / 32);
  p.rows = L->hidden;
  p.cols = L->inter;
  p.n_experts = L->n_experts;
  p.top_k = L->top_k;
  p.aq = hq;
  p.as = hs;
  p.route = route_view(L, ws, lay);
  p.rw = rw;
  float* partial = (float*)((uint8_t*)ws + lay.partial);
  p.partial = partial;
  int slots = L->n_experts + 1;
  if (T * L->top_k + 1 < slots) slots = T * L->top_k + 1;
  int rc = hip_rc(launch_prefill(false, p, slots, s));
  if (rc) return rc;
  return hip_rc(launch_combine(partial, T, L->top_k, L->hidden, y, s));
}

int forward(const moeq_layer* L, const void* x, const int32_t* ids, const float* rw, int T, float* y, void* ws,
            const WsLayout& lay, hipStream_t s);

// ---------------------------------------------------------------- allocation-free scratch
// Device memory of moeq_expert_forward_noalloc: a file-scope array that each GPU
// holds for the life of the process (no hipMalloc on any call). Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address is taken once per device with hipGetSymbolAddress,
// with that device current, and kept here.
__device__ __align__(256) uint8_t scratch[MOEQ_NOALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SCRATCH_MAX_DEVICES];

int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return MOEQ_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOEQ_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOEQ_OK;
}

}  // namespace

extern "C" {

int moeq_abi_version(void) { return MOEQ_ABI_VERSION; }

const char* moeq_status_string(int status) {
  switch (status) {
    case MOEQ_OK: return "ok";
    case MOEQ_E_INVAL: return "invalid argument";
    case MOEQ_E_FMT: return "unknown or unsupported format";
    case MOEQ_E_ALIGN: return "pointer or stride not aligned";
    case MOEQ_E_SHAPE: return "unsupported shape";
    case MOEQ_E_WORKSPACE: return "workspace missing or too small";
    case MOEQ_E_HIP: return "HIP launch or runtime error";
    case MOEQ_E_LOSSY: return "conversion would not be exact";
    case MOEQ_E_SCRATCH: return "workspace needed exceeds the allocation-free scratch (MOEQ_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

size_t moeq_plane_bytes(int fmt, int rows, int cols, int plane) { return plane_bytes(fmt, rows, cols, plane); }

size_t moeq_packed_bytes(int fmt, int rows, int cols) {
  size_t a = plane_bytes(fmt, rows, cols, 0), b = plane_bytes(fmt, rows, cols, 1);
  if (!a || !b) return 0;
  return a + b + (fmt == MOEQ_FMT_NVFP4 ? 4 : 0);
}

int moeq_pack_ggml(int fmt, const void* blocks_host, int rows, int cols, void* data_host, void* scales_host) {
  if (fmt != MOEQ_FMT_Q2_K && fmt != MOEQ_FMT_IQ2_XXS) return MOEQ_E_FMT;
  if (!blocks_host || !data_host || !scales_host) return MOEQ_E_INVAL;
  if (plane_bytes(fmt, rows, cols, 0) == 0) return MOEQ_E_SHAPE;
  const size_t nblk = (size_t)rows * (cols / 256);
  const uint8_t* src = (const uint8_t*)blocks_host;
  uint8_t* d = (uint8_t*)data_host;
  uint8_t* c = (uint8_t*)scales_host;
  for (size_t b = 0; b < nblk; b++) {
    if (fmt == MOEQ_FMT_Q2_K) {
      const uint8_t* s = src + b * 84;
      memcpy(d + b * 64, s + 16, 64);
      memcpy(c + b * 20, s, 16);
      memcpy(c + b * 20 + 16, s + 80, 4);
    } else {
      const uint8_t* s = src + b * 66;
      memcpy(d + b * 64, s + 2, 64);
      memcpy(c + b * 2, s, 2);
    }
  }
  return MOEQ_OK;
}

int moeq_pack_ggml_device(int fmt, const void* blocks, int rows, int cols, int n, void* data, void* scales,
                          void* stream) {
  if (fmt != MOEQ_FMT_Q2_K && fmt != MOEQ_FMT_IQ2_XXS) return MOEQ_E_FMT;
  if (!blocks || !data || !scales || n < 0) return MOEQ_E_INVAL;
  if (plane_bytes(fmt, rows, cols, 0) == 0) return MOEQ_E_SHAPE;
  if (n == 0) return MOEQ_OK;
  return hip_rc(launch_pack(fmt, (const uint8_t*)blocks, rows, cols, n, (uint8_t*)data, (uint8_t*)scales, S(stream)));
}

int moeq_mxfp4_to_nvfp4(const uint8_t* nib_host, const uint8_t* e8m0_host, int rows, int cols, uint8_t* nib_out_host,
                        uint8_t* e4m3_out_host, float* scale2_out_host) {
  if (!nib_host || !e8m0_host || !nib_out_host || !e4m3_out_host || !scale2_out_host) return MOEQ_E_INVAL;
  if (rows <= 0 || cols <= 0 || cols % 32) return MOEQ_E_SHAPE;
  const size_t nblk = (size_t)rows * (cols / 32);
  int emin = 255, emax = 0;
  for (size_t i = 0; i < nblk; i++) {
    int E = e8m0_host[i];
    if (E == 255) return MOEQ_E_LOSSY;
    emin = E < emin ? E : emin;
    emax = E > emax ? E : emax;
  }
  if (emax - emin > 17) return MOEQ_E_LOSSY;
  // Largest block exponent -> e4m3's largest power of two 2^8.
  *scale2_out_host = ldexpf(1.0f, emax - 127 - 8);
  for (size_t i = 0; i < nblk; i++) {
    int k = (int)e8m0_host[i] - emax + 8;  // -9 .. 8
    uint8_t code = k >= -6 ? (uint8_t)((k + 7) << 3) : (uint8_t)(1u << (k + 9));
    e4m3_out_host[2 * i] = code;
    e4m3_out_host[2 * i + 1] = code;
  }
  memcpy(nib_out_host, nib_host, (size_t)rows * cols / 2);
  return MOEQ_OK;
}

int moeq_mxfp8_to_tiled(const void* data, const void* scales, int rows, int cols, int n, void* tdata, void* tscales,
                        void* stream) {
  if (!data || !scales || !tdata || !tscales || n < 0) return MOEQ_E_INVAL;
  if (plane_bytes(MOEQ_FMT_MXFP8_TILED, rows, cols, 0) == 0) return MOEQ_E_SHAPE;
  if (!aligned(data, 16) || !aligned(tdata, 16) || !aligned(tscales, 4)) return MOEQ_E_ALIGN;
  if (n == 0) return MOEQ_OK;
  return hip_rc(launch_mxfp8_tile((const uint8_t*)data, (const uint8_t*)scales, rows, cols, n, (uint8_t*)tdata,
                                  (uint8_t*)tscales, S(stream)));
}

int moeq_mxfp4_to_nvfp4_device(const uint8_t* nib, const uint8_t* e8m0, int rows, int cols, int n, uint8_t* nib_out,
                               uint8_t* e4m3_out, float* scale2_out, uint32_t* status, void* stream) {
  if (!nib || !e8m0 || !nib_out || !e4m3_out || !scale2_out || !status || n < 0) return MOEQ_E_INVAL;
  if (rows <= 0 || cols <= 0 || cols % 32) return MOEQ_E_SHAPE;
  if (!aligned(nib, 16) || !aligned(nib_out, 16) || !aligned(scale2_out, 4) || !aligned(status, 4)) return MOEQ_E_ALIGN;
  if (n == 0) return MOEQ_OK;
  return hip_rc(launch_mx4_to_nv4(nib, e8m0, rows, cols, n, nib_out, e4m3_out, scale2_out, status, S(stream)));
}

int moeq_nvfp4_to_mxfp4_device(const uint8_t* nib, const uint8_t* e4m3, const float* scale2, int rows, int cols, int n,
                               uint8_t* nib_out, uint8_t* e8m0_out, uint32_t* status, void* stream) {
  if (!nib || !e4m3 || !scale2 || !nib_out || !e8m0_out || !status || n < 0) return MOEQ_E_INVAL;
  if (rows <= 0 || cols <= 0 || cols % 32) return MOEQ_E_SHAPE;
  if (!aligned(nib, 16) || !aligned(nib_out, 16) || !aligned(scale2, 4) || !aligned(status, 4)) return MOEQ_E_ALIGN;
  if (n == 0) return MOEQ_OK;
  return hip_rc(launch_nv4_to_mx4(nib, e4m3, scale2, rows, cols, n, nib_out, e8m0_out, status, S(stream)));
}

int moeq_dequant(const moeq_weight* w, int expert, float* out, void* stream) {
  int rc = check_weight(w, false);
  if (rc) return rc;
  if (expert < 0 || expert >= w->n_experts) return MOEQ_E_INVAL;
  if (!out) return MOEQ_E_INVAL;
  if (!aligned(out, 4)) return MOEQ_E_ALIGN;
  return hip_rc(launch_dequant(w->fmt, ref_of(*w), w->grid, w->rows, w->cols, expert, out, S(stream)));
}

size_t moeq_workspace_bytes(const moeq_layer* L, int T) {
  if (check_layer(L) || T < 0) return 0;
  return ws_layout(L, T).total;
}

int moeq_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes < 256) return MOEQ_E_WORKSPACE;
  if (!aligned(ws, 256)) return MOEQ_E_ALIGN;
  return hip_rc(launch_clear_words((uint32_t*)ws, 64, S(stream)));
}

int moeq_route(const moeq_layer* L, const int32_t* ids, int T, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (T < 0 || !ids) return MOEQ_E_INVAL;
  if ((rc = check_ws(L, T, ws, ws_bytes))) return rc;
  if (T == 0) return MOEQ_OK;
  WsLayout lay = ws_layout(L, T);
  return hip_rc(launch_route(ids, T * L->top_k, L->n_experts, route_view(L, ws, lay), err_word(ws), S(stream)));
}

int moeq_gate_up(const moeq_layer* L, const void* x, const int32_t* ids, int T, float* h, void* ws, size_t ws_bytes,
                 void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (T < 0 || !x || !ids || !h) return MOEQ_E_INVAL;
  if (!aligned(x, 16) || !aligned(h, 16)) return MOEQ_E_ALIGN;
  if ((rc = check_ws(L, T, ws, ws_bytes))) return rc;
  if (T == 0) return MOEQ_OK;
  return run_gate_up(L, x, ids, T, h, ws, ws_layout(L, T), S(stream));
}

int moeq_gate_up_timed(const moeq_layer* L, const void* x, const int32_t* ids, int T, float* h, void* ws,
                       size_t ws_bytes, void* stream, void* start_event, void* stop_event) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (T < 0 || !x || !ids || !h) return MOEQ_E_INVAL;
  if (!aligned(x, 16) || !aligned(h, 16)) return MOEQ_E_ALIGN;
  if ((rc = check_ws(L, T, ws, ws_bytes))) return rc;
  if (T == 0) return MOEQ_OK;
  LaunchEvents ev{(hipEvent_t)start_event, (hipEvent_t)stop_event};
  return run_gate_up(L, x, ids, T, h, ws, ws_layout(L, T), S(stream), &ev);
}

int moeq_down(const moeq_layer* L, const float* h, const int32_t* ids, const float* rw, int T, float* y, void* ws,
              size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (T < 0 || !h || !ids || !rw || !y) return MOEQ_E_INVAL;
  if (!aligned(h, 16) || !aligned(y, 16)) return MOEQ_E_ALIGN;
  if ((rc = check_ws(L, T, ws, ws_bytes))) return rc;
  if (T == 0) return MOEQ_OK;
  return run_down(L, h, ids, rw, T, y, ws, ws_layout(L, T), S(stream));
}

int moeq_expert_forward(const moeq_layer* L, const void* x, const int32_t* ids, const float* rw, int T, float* y,
                        void* ws, size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (T < 0 || !x || !ids || !rw || !y) return MOEQ_E_INVAL;
  if (!aligned(x, 16) || !aligned(y, 16)) return MOEQ_E_ALIGN;
  if ((rc = check_ws(L, T, ws, ws_bytes))) return rc;
  if (T == 0) return MOEQ_OK;
  return forward(L, x, ids, rw, T, y, ws, ws_layout(L, T), S(stream));
}

int moeq_expert_forward_noalloc(const moeq_layer* L, const void* x, const int32_t* ids, const float* rw, int T,
                                float* y, uint32_t* dev_err, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (T < 0 || !x || !ids || !rw || !y) return MOEQ_E_INVAL;
  if (!aligned(x, 16) || !aligned(y, 16) || (dev_err && !aligned(dev_err, 4))) return MOEQ_E_ALIGN;
  WsLayout lay = ws_layout(L, T);
  if (lay.total > MOEQ_NOALLOC_SCRATCH_BYTES) return MOEQ_E_SCRATCH;
  if (T == 0) return MOEQ_OK;
  void* ws = nullptr;
  if ((rc = noalloc_scratch(&ws))) return rc;
  lay.err = dev_err;  // null: the scratch's own word, which nothing reads
  return forward(L, x, ids, rw, T, y, ws, lay, S(stream));
}

}  // extern "C"

namespace {

int forward(const moeq_layer* L, const void* x, const int32_t* ids, const float* rw, int T, float* y, void* ws,
            const WsLayout& lay, hipStream_t s) {
  int rc;
  float* h = (float*)((uint8_t*)ws + lay.h);
  if (T > 1 && !(gu_direct(L, T) && dn_direct(L, T, h))) {
    rc = hip_rc(launch_route(ids, T * L->top_k, L->n_experts, route_view(L, ws, lay), err_of(ws, lay), s));
    if (rc) return rc;
  }
  const bool pf = prefill_buffers(L, T) && prefill_a_fits(L, T);
  const bool gu_pf = pf && check_prefill(L, true) == MOEQ_OK;
  const bool dn_pf = pf && check_prefill(L, false) == MOEQ_OK;
  uint8_t* xq = (uint8_t*)ws + lay.xq;
  uint8_t* xs = (uint8_t*)ws + lay.xs;
  uint8_t* hq = (uint8_t*)ws + lay.hq;
  uint8_t* hs = (uint8_t*)ws + lay.hs;
  if (gu_pf) {  // W4A8: MXFP8 x; fp32 h too when the down projection needs it
    if ((rc = hip_rc(launch_quant_mxfp8(0, x, T, L->hidden, xq, xs, s)))) return rc;
    if ((rc = run_prefill_gate_up(L, xq, xs, T, dn_pf ? nullptr : h, hq, hs, ws, lay, s))) return rc;
  } else if ((rc = run_gate_up(L, x, ids, T, h, ws, lay, s))) {
    return rc;
  }
  if (dn_pf) {  // W4A8: MXFP8 h (quantised here when the gate/up produced fp32)
    if (!gu_pf && (rc = hip_rc(launch_quant_mxfp8(1, h, T * L->top_k, L->inter, hq, hs, s)))) return rc;
    return run_prefill_down(L, hq, hs, rw, T, y, ws, lay, s);
  }
  return run_down(L, h, ids, rw, T, y, ws, lay, s);
}

}  // namespace

extern "C" {

int moeq_prefill_gate_up(const moeq_layer* L, const uint8_t* xq, const uint8_t* xs, const int32_t* ids, int T,
                         float* h_f32, uint8_t* hq, uint8_t* hs, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if ((rc = check_prefill(L, true))) return rc;
  if (T < 0 || !xq || !xs || !ids || !hq || !hs) return MOEQ_E_INVAL;
  if (!aligned(xq, 16) || !aligned(xs, 8) || (h_f32 && !aligned(h_f32, 4))) return MOEQ_E_ALIGN;
  if ((rc = check_ws(L, T, ws, ws_bytes))) return rc;
  if (T == 0) return MOEQ_OK;
  return run_prefill_gate_up(L, xq, xs, T, h_f32, hq, hs, ws, ws_layout(L, T), S(stream));
}

int moeq_prefill_down(const moeq_layer* L, const uint8_t* hq, const uint8_t* hs, const int32_t* ids, const float* rw,
                      int T, float* y, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if ((rc = check_prefill(L, false))) return rc;
  if (T < 0 || !hq || !hs || !ids || !rw || !y) return MOEQ_E_INVAL;
  if (!aligned(hq, 16) || !aligned(hs, 8) || !aligned(y, 16)) return MOEQ_E_ALIGN;
  if ((rc = check_ws(L, T, ws, ws_bytes))) return rc;
  if (T == 0) return MOEQ_OK;
  if (T < 2) return MOEQ_E_SHAPE;  // the combine buffer exists for T > 1
  return run_prefill_down(L, hq, hs, rw, T, y, ws, ws_layout(L, T), S(stream));
}

int moeq_linear(const moeq_weight* w, int expert, const void* x, int T, float* y, void* stream) {
  int rc = check_weight(w, false);
  if (rc) return rc;
  const bool mx8 = dense_only(w->fmt);
  if (mx8 && !linear_mx8_fits(w->fmt, w->rows, w->cols)) return MOEQ_E_SHAPE;
  const bool mfma = w->fmt == MOEQ_FMT_FP8_B128 && T > 1 && linear_fp8_fits(w->rows, w->cols);
  int lpr, cpl;
  if (!mx8 && !mfma && !chunk_geometry(w->fmt, w->cols, &lpr, &cpl)) return MOEQ_E_SHAPE;
  if (expert < 0 || expert >= w->n_experts || T < 0 || !x || !y) return MOEQ_E_INVAL;
  if (!aligned(x, 16) || !aligned(y, 4)) return MOEQ_E_ALIGN;
  if (w->cols % 8) return MOEQ_E_SHAPE;
  if (T == 0) return MOEQ_OK;
  if (mx8) {
    Mx8Params mp;
    mp.w = static_cast<const uint8_t*>(w->data) + (size_t)expert * w->expert_stride;
    mp.s = static_cast<const uint8_t*>(w->scales) + (size_t)expert * w->scale_expert_stride;
    mp.x = static_cast<const uint16_t*>(x);
    mp.y = y;
    mp.rows = w->rows;
    mp.cols = w->cols;
    mp.T = T;
    return hip_rc(launch_linear_mx8(w->fmt, mp, S(stream)));
  }
  if (mfma) {
    LinearParams lp;
    lp.w = static_cast<const uint8_t*>(w->data) + (size_t)expert * w->expert_stride;
    lp.s = static_cast<const uint8_t*>(w->scales) + (size_t)expert * w->scale_expert_stride;
    lp.x = static_cast<const uint16_t*>(x);
    lp.y = y;
    lp.rows = w->rows;
    lp.cols = w->cols;
    lp.T = T;
    return hip_rc(launch_linear_fp8(lp, S(stream)));
  }
  WsLayout lay;
  memset(&lay, 0, sizeof(lay));
  GemvParams p = gemv_params(nullptr, *w, nullptr, nullptr, lay);
  p.act = x;
  p.T = T;
  p.expert = expert;
  p.mode = MODE_LINEAR;
  p.out = y;
  return hip_rc(launch_gemv(w->fmt, EPI_PLAIN, p, 1, T > 1 ? 4 : 1, S(stream)));
}

int moeq_quantize_mxfp8(const void* x, int T, int K, uint8_t* q, uint8_t* e8m0, void* stream) {
  if (!x || !q || !e8m0 || T < 0) return MOEQ_E_INVAL;
  if (K <= 0 || K % 32) return MOEQ_E_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 16)) return MOEQ_E_ALIGN;
  if (T == 0) return MOEQ_OK;
  return hip_rc(launch_quant_mxfp8(0, x, T, K, q, e8m0, S(stream)));
}

int moeq_quantize_mxfp8_f32(const float* x, int T, int K, uint8_t* q, uint8_t* e8m0, void* stream) {
  if (!x || !q || !e8m0 || T < 0) return MOEQ_E_INVAL;
  if (K <= 0 || K % 32) return MOEQ_E_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 16)) return MOEQ_E_ALIGN;
  if (T == 0) return MOEQ_OK;
  return hip_rc(launch_quant_mxfp8(1, x, T, K, q, e8m0, S(stream)));
}

int moeq_check_device_error(void* ws, void* stream, uint32_t* err_host, int clear) {
  if (!ws || !err_host) return MOEQ_E_INVAL;
  hipStream_t s = S(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return MOEQ_E_HIP;
  if (hipMemcpy(err_host, ws, 4, hipMemcpyDeviceToHost) != hipSuccess) return MOEQ_E_HIP;
  if (clear) {
    if (launch_clear_words((uint32_t*)ws, 1, s) != hipSuccess) return MOEQ_E_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return MOEQ_E_HIP;
  }
  return MOEQ_OK;
}

}  // extern "C"
