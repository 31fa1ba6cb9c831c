// Kernel parameter blocks and host-side launchers shared by the kernel sources
// and the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moeq {

enum { MODE_DIRECT = 0, MODE_GROUPED = 1, MODE_LINEAR = 2 };
enum { EPI_SWIGLU = 0, EPI_PARTIAL = 1, EPI_PLAIN = 2 };

// Routing block inside the workspace (int32 words):
//   [0]                n_slots (touched experts, plus one slot for invalid ids if any)
//   [1, E + 2)         slot -> expert (E marks the bucket of out-of-range ids)
//   [E + 2, 2E + 4)    bucket offsets into perm (bucket E = out-of-range ids)
//   [2E + 4, ...)      perm: pair indices grouped by expert
// Tokens per prefill work item (two 32-row tiles of the matrix instruction).
constexpr int PREFILL_MC = 64;

struct RouteView {
  int32_t* base;
  int E, P;  // experts, (token, slot) pairs
  __host__ __device__ int32_t* n_slots() const { return base; }
  __host__ __device__ int32_t* slots() const { return base + 1; }
  __host__ __device__ int32_t* offsets() const { return base + E + 2; }
  __host__ __device__ int32_t* perm() const { return base + 2 * E + 4; }
  // Prefill work items: one per PREFILL_MC pairs of a bucket (bucket E holds the
  // out-of-range ids), in bucket order: item q covers pairs chunk_m0[q] ..
  // chunk_m0[q] + PREFILL_MC - 1 of bucket chunk_e[q].
  __host__ __device__ int32_t* n_chunks() const { return base + 2 * E + 4 + P; }
  __host__ __device__ int32_t* chunk_e() const { return base + 2 * E + 5 + P; }
  __host__ __device__ int32_t* chunk_m0() const { return base + 2 * E + 5 + P + max_chunks(E, P); }
  // sum over buckets of ceil(count / MC) <= P / MC + (non-empty buckets)
  __host__ __device__ static int max_chunks(int E, int P) { return P / PREFILL_MC + (P < E + 1 ? P : E + 1); }
  static size_t words(int E, int P) { return (size_t)(2 * E + 5 + P) + 2 * (size_t)max_chunks(E, P); }
};

struct WeightRef {
  const uint8_t* data;
  const uint8_t* scales;
  size_t estride, sestride;
  const float* scale2;  // NVFP4 per-expert scale_2 or nullptr
};

struct GemvParams {
  WeightRef w[2];
  const uint8_t* grid;  // IQ2_XXS codebook
  int rows, cols, n_experts, lpr, chunks;
  const void* act;      // bf16 [tokens][cols] or fp32 [pairs][cols]
  int mode, T, top_k, expert;
  const int32_t* ids;
  RouteView route;
  const float* rw;
  float* out;
  uint32_t* err;
  int rows_per_wg, U;
};

struct Down1Params {
  WeightRef w;
  const uint8_t* grid;
  int rows, cols, n_experts, lpr, chunks, top_k;
  int T;           // tokens (the MXFP4 matrix-unit kernel takes one per grid row; 0 or 1 elsewhere)
  const float* h;  // fp32 [T][top_k][cols]
  const int32_t* ids;
  const float* rw;
  float* y;
  uint32_t* err;
  int rows_per_wg, U;
};


struct PrefillParams {
  WeightRef w[2];        // gate/up pass: gate, up; down pass: down (w[0])
  int rows, cols;        // weight shape: N x K
  int n_experts, top_k;
  const uint8_t* aq;     // A codes [*][cols]: xq rows indexed by token (gate/up) or hq rows by pair (down)
  const uint8_t* as;     // A e8m0 [*][cols/32]
  RouteView route;
  const float* rw;
  float* h_f32;          // gate/up: optional fp32 h [pairs][rows]
  uint8_t* hq;           // gate/up: MXFP8 h codes [pairs][rows]
  uint8_t* hs;           // gate/up: e8m0 [pairs][rows/32]
  float* partial;        // down: [pairs][rows]
};

// Dense FP8 block-128 linear on the bf16 matrix instruction (two or more tokens).
struct LinearParams {
  const uint8_t* w;   // E4M3 codes [rows][cols] of one expert
  const uint8_t* s;   // e8m0 [rows/128][cols/128]
  const uint16_t* x;  // bf16 [T][cols], 16-byte aligned
  float* y;           // fp32 [T][rows]
  int rows, cols, T;
};

// Dense FP8 linear with power-of-two block scales on the block-scaled matrix
// instruction (MXFP8, MXFP8 pre-stored in the operand order, FP8 block-32).
struct Mx8Params {
  const uint8_t* w;   // E4M3 codes of one expert (row-major, or the pre-stored order)
  const uint8_t* s;   // its e8m0 scale plane
  const uint16_t* x;  // bf16 [T][cols], 16-byte aligned
  float* y;           // fp32 [T][rows]
  int rows, cols, T;
};

// Launchers (return hipError_t of the launch).
hipError_t launch_dequant(int fmt, const WeightRef& w, const uint8_t* grid, int rows, int cols, int expert, float* out,
                          hipStream_t s);
// start/stop (hipEvent_t, may be null): recorded at the kernel's own start and end.
struct LaunchEvents {
  hipEvent_t start, stop;
};
hipError_t launch_gemv(int fmt, int epi, const GemvParams& p, int n_slots, int mt, hipStream_t s,
                       const LaunchEvents* ev = nullptr);
hipError_t launch_down1(int fmt, const Down1Params& p, hipStream_t s);
hipError_t launch_route(const int32_t* ids, int P, int E, RouteView rv, uint32_t* err, hipStream_t s);
hipError_t launch_combine(const float* partial, int T, int K, int H, float* y, hipStream_t s);
hipError_t launch_quant_mxfp8(int in_f32, const void* x, int T, int K, uint8_t* q, uint8_t* e, hipStream_t s);
hipError_t launch_pack(int fmt, const uint8_t* blocks, int rows, int cols, int n, uint8_t* data, uint8_t* scales,
                       hipStream_t s);
hipError_t launch_clear_words(uint32_t* p, int n, hipStream_t s);
hipError_t launch_prefill(bool gate_up, const PrefillParams& p, int n_slots, hipStream_t s);
bool gu1_mx4_fits(int rows, int cols);  // cols % 512 == 0, cols <= 4096
// Single-token gate/up + SwiGLU for MXFP4 or NVFP4 on the block-scaled matrix instruction.
hipError_t launch_gu1_fp4(int fmt, const GemvParams& p, int n_slots, hipStream_t s, const LaunchEvents* ev);
bool down1_mx4_fits(int rows, int cols, int top_k);  // cols % 512 == 0, cols <= 2048, top_k <= 8
// Single-token down + weighted combine for MXFP4 on the block-scaled matrix instruction.
hipError_t launch_down1_mx4(const Down1Params& p, hipStream_t s);
bool down1_q2k_fits(int rows, int cols, int top_k);  // cols % 256 == 0, cols <= 2048, top_k <= 6
// Q2_K down + weighted combine of one token per grid row (p.T rows) on the
// block-scaled FP8 matrix instruction.
hipError_t launch_down1_q2k(const Down1Params& p, hipStream_t s);
// Token-grouped Q2_K down (T > 1) on the block-scaled FP8 matrix instruction: h
// (p.act, fp32 [pairs][cols], 16-byte aligned) to digit planes in dq / dsc
// (dn_q2k_g_digit_bytes / dn_q2k_g_scale_bytes), then route-weighted partials
// [pairs][rows] for the combine.
bool dn_q2k_g_fits(int rows, int cols);  // cols % 256 == 0, cols <= 2048
size_t dn_q2k_g_digit_bytes(long pairs, int cols);
size_t dn_q2k_g_scale_bytes(long pairs, int cols);
hipError_t launch_dn_q2k_g(const GemvParams& p, int n_slots, uint8_t* dq, uint8_t* dsc, hipStream_t s);
// Token-grouped Q2_K down (T > 1) on the bf16 matrix instruction: route-weighted
// partials [pairs][rows] for the combine.
bool dn_q2k_fits(int rows, int cols, long pairs);
hipError_t launch_dn_q2k(const GemvParams& p, int n_slots, hipStream_t s);
// Token-grouped IQ2_XXS down (T > 1) on the bf16 matrix instruction (same shape
// conditions as the Q2_K one).
hipError_t launch_dn_iq2(const GemvParams& p, int n_slots, hipStream_t s);
bool gu_iq2_fits(int rows, int cols);  // cols % 256 == 0
// Grouped gate/up + SwiGLU for IQ2_XXS on the bf16 matrix instruction (T > 1).
// wide: decode each superblock once for two 16-token tiles (many tokens per expert).
hipError_t launch_gu_iq2(const GemvParams& p, int n_slots, bool wide, hipStream_t s);
bool linear_fp8_fits(int rows, int cols);  // rows % 128 == 0, cols % 256 == 0
hipError_t launch_linear_fp8(const LinearParams& p, hipStream_t s);

// Batched (T > 1) MXFP4 gate/up + SwiGLU and down partials on the block-scaled
// matrix instruction, each routed expert's weights read once per step.
bool gu_mx4_g_fits(int rows, int cols);  // cols % 512 == 0, cols <= 4096
bool dn_mx4_g_fits(int rows, int cols);  // cols % 512 == 0, cols <= 2048
hipError_t launch_gu_fp4_g(int fmt, const GemvParams& p, int n_slots, hipStream_t s);  // MXFP4 or NVFP4
hipError_t launch_dn_mx4_g(const GemvParams& p, int n_slots, hipStream_t s);

bool linear_mx8_fits(int fmt, int rows, int cols);  // rows % 16, cols % 128 (pre-stored: % 512), cols <= 8192
hipError_t launch_linear_mx8(int fmt, const Mx8Params& p, hipStream_t s);
// Row-major MXFP8 -> the pre-stored operand order, n tensors back to back.
hipError_t launch_mxfp8_tile(const uint8_t* data, const uint8_t* scales, int rows, int cols, int n, uint8_t* tdata,
                             uint8_t* tscales, hipStream_t s);
// MXFP4 <-> NVFP4 scale re-encodes of n tensors back to back (status[i] = 1: not exact, outputs untouched).
hipError_t launch_mx4_to_nv4(const uint8_t* nib, const uint8_t* e8m0, int rows, int cols, int n, uint8_t* nib_out,
                             uint8_t* e4m3_out, float* scale2_out, uint32_t* status, hipStream_t s);
hipError_t launch_nv4_to_mx4(const uint8_t* nib, const uint8_t* e4m3, const float* scale2, int rows, int cols, int n,
                             uint8_t* nib_out, uint8_t* e8m0_out, uint32_t* status, hipStream_t s);

// Chunk geometry: weights per 16-byte chunk; lanes per row and chunks per lane.
int weights_per_chunk(int fmt);
bool chunk_geometry(int fmt, int cols, int* lpr, int* cpl);

}  // namespace moeq
