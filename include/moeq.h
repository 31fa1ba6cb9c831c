/*
 * moeq.h - C ABI of the MI355X (gfx950) block-quantized routed-MoE library.
 *
 * The library computes the routed-expert projection of a DeepSeek-V4-Flash-shaped
 * MoE layer (DeepSeek-V4-Flash W4A16-FP8 model card, "Architecture & precision",
 * base-model table: 256 routed experts, top-6, hidden 4096, 43 layers) with expert
 * weights in block-quantized formats, on one GPU:
 *
 *   for token t routed to experts e_k with route weights w_k (k < top_k):
 *     h_k = silu(G_e x_t) * (U_e x_t),   y_t = sum_k w_k * (D_e h_k)
 *
 * At decode (few tokens) each projection streams the routed experts' weights:
 * MXFP4 and NVFP4 gate/up and MXFP4 down feed the FP4 codes straight into the
 * block-scaled matrix instruction, and the Q2_K down its 2-bit codes as FP8
 * operands of the same instruction; IQ2_XXS and the remaining shapes decode on the
 * VALU (dequantize + GEMV). Up to 8 tokens (4 for NVFP4 gate/up; Q2_K down below
 * 1.06 pairs per touched expert) these kernels run over every (token, slot) pair
 * with no routing step; beyond, each routed expert is read once per step for all
 * of its tokens (MXFP4, the NVFP4 gate/up and the Q2_K down on the block-scaled
 * instruction, Q2_K's sub-block scale and min folded into the FP8 operand; IQ2_XXS
 * gate/up and down decoding once per 16-token tile for the bf16 matrix
 * instruction). At prefill with MXFP4 weights it is a token-grouped GEMM
 * on the block-scaled FP4 matrix instructions, with activations quantised to
 * MXFP8 (fp4 weights times E4M3 activations: DeepSeekv4 Flash for 1x Spark forum
 * thread, second post). The decode paths agree with the exact layer to the
 * documented tolerance, the prefill path with the same layer on MXFP8
 * activations; which path runs depends only on formats, shapes, T and
 * alignment, never on the data.
 *
 * Conventions for every entry point:
 *  - Pointers named *_host are host memory; every other buffer pointer is device
 *    memory on the current HIP device, owned and allocated by the caller. The
 *    library never allocates, frees or synchronises on the forward path and keeps
 *    no global state; launches are asynchronous on `stream` (a hipStream_t passed
 *    as void*, NULL = the default stream) and may be captured into a HIP graph.
 *  - Arguments are checked on the host before any launch; a check that fails
 *    returns a negative MOEQ_E_* code and launches nothing. MOEQ_E_HIP reports a
 *    launch error. Faults inside kernels follow HIP semantics (reported at the
 *    next synchronisation). Expert ids outside [0, n_experts) never cause an
 *    out-of-bounds access: the pair is skipped (its outputs are zero) and
 *    MOEQ_DEVERR_EXPERT_ID is set in the workspace's device error word.
 *  - Element order: rows are output features, cols are input features (the
 *    contraction axis); all matrices are row-major.
 */
#ifndef MOEQ_H_
#define MOEQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOEQ_ABI_VERSION 2

/* ------------------------------------------------------------------ formats
 * Device layout of one expert tensor [rows, cols] (the `data` and `scales`
 * planes of moeq_weight; experts are expert_stride / scale_expert_stride bytes
 * apart):
 *
 * MOEQ_FMT_MXFP4 - e2m1 elements, one e8m0 scale per 32 along cols (REAP K180
 *   Mixed NVFP4 card, lossless MXFP4 -> NVFP4 conversion section; 4.25 bits per
 *   weight in the 1x Spark forum thread, first post).
 *   data: u8 [rows][cols/2], element 2j in the low nibble of byte j.
 *   scales: u8 [rows][cols/32] e8m0 codes; weight = e2m1 * 2^(E-127), E=255 NaN.
 * MOEQ_FMT_NVFP4 - e2m1 elements, one e4m3 scale per 16, one fp32 scale_2 per
 *   expert tensor (same card, "Why this mix?": 4.50 bits per weight).
 *   data: as MXFP4. scales: u8 [rows][cols/16] e4m3fn codes.
 *   scale2: fp32 [n_experts]. weight = e2m1 * e4m3 * scale_2.
 * MOEQ_FMT_Q2_K - ggml 256-weight superblocks, 84 bytes (2.625 bits per weight;
 *   IQ2_XXS + Q2_K + FP8 hybrid card, format table). Stored as two planes so
 *   every load is aligned; moeq_pack_ggml converts from the contiguous block.
 *   data: u8 [rows][cols/256][64] = the block's qs bytes.
 *   scales: u8 [rows][cols/256][20] = the block's 16 scale bytes, then d and
 *   dmin (fp16, little-endian).
 *   weight i of a superblock: j = i/16, h = i/128, r = i%128,
 *   q = (qs[32h + r%32] >> 2*(r/32)) & 3,
 *   w = d * (sc[j] & 15) * q - dmin * (sc[j] >> 4).
 * MOEQ_FMT_IQ2_XXS - ggml 256-weight superblocks, 66 bytes (2.0625 bits per
 *   weight; same table). Two planes:
 *   data: u8 [rows][cols/256][64] = 8 sub-blocks of (u32 a0, u32 a1).
 *   scales: fp16 d [rows][cols/256].
 *   grid: u8 [256][8] device codebook (an input: any values 0..255).
 *   weight 32b + 8l + j: db = d * (0.5 + (a1 >> 28)) / 4,
 *   g = grid[(a0 >> 8l) & 255][j], c = (a1 >> 7l) & 127,
 *   mask = c | parity(c) << 7, w = (mask >> j & 1 ? -1 : 1) * db * g.
 * MOEQ_FMT_FP8_B128 - E4M3 weights with one UE8M0 scale per 128x128 tile (IQ2_XXS
 *   + Q2_K + FP8 hybrid card, format table; W4A16-FP8 card, FP8 block 128x128).
 *   data: u8 [rows][cols] e4m3fn codes. scales: u8 [rows/128][cols/128].
 *
 * Dense-linear formats (moeq_linear and moeq_dequant only; a layer using one is
 * refused with MOEQ_E_FMT):
 * MOEQ_FMT_FP8_B32 - E4M3 weights with one UE8M0 scale per 32x32 tile, the dense
 *   FP8 weights of DeepSeek-V4.1 (DeepSeek-V4.1-Flash mixed-Q2 GGUF card, Recipe:
 *   V4.1 uses 32x32 E8M0 block scales, V4 128x128; reading one as the other
 *   rescales every weight). data: u8 [rows][cols]; scales: u8 [rows/32][cols/32].
 * MOEQ_FMT_MXFP8 - E4M3 elements with one e8m0 scale per 32 along cols (8.25 bits
 *   per weight), the checkpoint's format for attention, shared experts and the head
 *   (DeepSeekv4 Flash for 1x Spark forum thread, first post).
 *   data: u8 [rows][cols]; scales: u8 [rows][cols/32]; weight = e4m3 * 2^(E-127).
 * MOEQ_FMT_MXFP8_TILED - the same bytes pre-stored in the order of the block-scaled
 *   matrix instruction's operand (same thread, second post: MXFP8 weights stored
 *   in the matrix engine's layout so that nothing is repacked at run time); rows a
 *   multiple of 16, cols of 512. Made from MOEQ_FMT_MXFP8 by moeq_mxfp8_to_tiled.
 *   data: per tile of 16 rows x 128 cols (tile = (r/16) * (cols/128) + c/128),
 *   2048 bytes at tile * 2048; lane L = n + 16g of the tile holds the 32 bytes at
 *   32 L: row n, cols 16g + [0, 16) then 64 + 16g + [0, 16) of the tile.
 *   scales: per group of 16 rows x 512 cols (group = (r/16) * (cols/512) +
 *   c/512), 256 bytes; byte 4 L + j = e8m0 of row n, 32-block 4j + g of the group.
 */
#define MOEQ_FMT_MXFP4 1
#define MOEQ_FMT_NVFP4 2
#define MOEQ_FMT_Q2_K 3
#define MOEQ_FMT_IQ2_XXS 4
#define MOEQ_FMT_FP8_B128 5
#define MOEQ_FMT_MXFP8 6
#define MOEQ_FMT_FP8_B32 7
#define MOEQ_FMT_MXFP8_TILED 8

/* ------------------------------------------------------------------ status */
#define MOEQ_OK 0
#define MOEQ_E_INVAL -1     /* null pointer, negative count, bad argument */
#define MOEQ_E_FMT -2       /* unknown format, or a format the entry point does not take */
#define MOEQ_E_ALIGN -3     /* pointer or stride not aligned as documented */
#define MOEQ_E_SHAPE -4     /* shape the format or the kernels cannot hold */
#define MOEQ_E_WORKSPACE -5 /* workspace missing or smaller than moeq_workspace_bytes */
#define MOEQ_E_HIP -6       /* a HIP call or kernel launch failed */
#define MOEQ_E_LOSSY -7     /* MXFP4 -> NVFP4 cannot be exact (span > 17 or NaN scale) */
#define MOEQ_E_SCRATCH -8   /* moeq_expert_forward_noalloc: the call needs more than the scratch holds */

/* Bits of the device error word (first 4 bytes of a workspace). */
#define MOEQ_DEVERR_EXPERT_ID 1u /* an expert id was outside [0, n_experts) */

/* ------------------------------------------------------------------ descriptors
 * Read on the host only, during the call. */
typedef struct moeq_weight {
  int fmt;                    /* MOEQ_FMT_* */
  int rows;                   /* output features */
  int cols;                   /* input features */
  int n_experts;              /* experts stored expert-major */
  const void* data;           /* 16-byte aligned */
  size_t expert_stride;       /* bytes between experts in data, multiple of 16 */
  const void* scales;         /* 4-byte aligned */
  size_t scale_expert_stride; /* bytes between experts in scales, multiple of 4 */
  const float* scale2;        /* NVFP4: fp32 [n_experts]; else ignored */
  const uint8_t* grid;        /* IQ2_XXS: u8 [256][8]; else ignored */
} moeq_weight;

typedef struct moeq_layer {
  int hidden;    /* H: gate/up cols, down rows */
  int inter;     /* I: gate/up rows, down cols */
  int n_experts; /* E */
  int top_k;     /* K, 1..16 */
  moeq_weight gate, up, down;
} moeq_layer;

/* ------------------------------------------------------------------ sizes */
int moeq_abi_version(void);
const char* moeq_status_string(int status);

/* Bytes of plane 0 (data) or plane 1 (scales) of one expert tensor [rows, cols];
 * 0 for an invalid format, plane or shape. cols must be a multiple of the format's
 * block: 32 MXFP4, 16 NVFP4, 256 Q2_K and IQ2_XXS, 128 FP8_B128 (rows too). */
size_t moeq_plane_bytes(int fmt, int rows, int cols, int plane);

/* Total bytes of one expert tensor, both planes plus NVFP4's 4-byte scale_2. The
 * algorithmic bytes per weight equal the format's bits per weight / 8. */
size_t moeq_packed_bytes(int fmt, int rows, int cols);

/* ------------------------------------------------------------------ host utilities */

/* Repack contiguous ggml blocks (Q2_K: 84 B, IQ2_XXS: 66 B per 256 weights, rows x
 * cols/256 blocks row-major) into the two device planes, in host memory. */
int moeq_pack_ggml(int fmt, const void* blocks_host, int rows, int cols, void* data_host, void* scales_host);

/* Device version over n tensors stored back to back (block bytes, data and scale
 * planes each contiguous per tensor). */
int moeq_pack_ggml_device(int fmt, const void* blocks, int rows, int cols, int n, void* data, void* scales,
                          void* stream);

/* Lossless MXFP4 -> NVFP4 re-encode of one tensor in host memory (REAP K180 Mixed
 * NVFP4 card, conversion section and "How It Was Built" step 3): nibbles copied,
 * e8m0 per 32 -> e4m3 per 16 with scale_2 = 2^(Emax-135), e4m3 = 2^(E-Emax+8).
 * MOEQ_E_LOSSY if Emax - Emin > 17 or a code is 255; outputs are then untouched. */
int moeq_mxfp4_to_nvfp4(const uint8_t* nib_host, const uint8_t* e8m0_host, int rows, int cols, uint8_t* nib_out_host,
                        uint8_t* e4m3_out_host, float* scale2_out_host);

/* Row-major MXFP8 (MOEQ_FMT_MXFP8) -> the pre-stored operand order
 * (MOEQ_FMT_MXFP8_TILED) for n tensors stored back to back in device memory
 * (data planes rows * cols bytes apart, scale planes rows * cols / 32). rows a
 * multiple of 16 and cols of 512 (MOEQ_E_SHAPE otherwise); data and tdata 16-byte
 * aligned, tscales 4-byte aligned; outputs must not overlap inputs. Asynchronous
 * on `stream`. */
int moeq_mxfp8_to_tiled(const void* data, const void* scales, int rows, int cols, int n, void* tdata, void* tscales,
                        void* stream);

/* Device versions of the MXFP4 <-> NVFP4 re-encodes (REAP K180 Mixed NVFP4 card,
 * conversion section and "How It Was Built" step 3; the rule is the host one above),
 * for n tensors [rows][cols] stored back to back in device memory: nibbles rows *
 * cols / 2 bytes apart, e8m0 planes rows * cols / 32, e4m3 planes rows * cols / 16,
 * one scale_2 per tensor. status (device, u32 [n]) receives 0 for a tensor
 * converted exactly and 1 for one that cannot be (MXFP4 -> NVFP4: exponent span
 * above 17 or a NaN scale; NVFP4 -> MXFP4: the two 16-halves of a block differ or
 * their scale times scale_2 is not a power of two 2^k, -127 <= k <= 127), whose
 * outputs are then left untouched. nib_out may equal nib (converted in place);
 * the scale planes must not overlap. Nibble planes 16-byte aligned. Asynchronous on
 * `stream`. */
int moeq_mxfp4_to_nvfp4_device(const uint8_t* nib, const uint8_t* e8m0, int rows, int cols, int n, uint8_t* nib_out,
                               uint8_t* e4m3_out, float* scale2_out, uint32_t* status, void* stream);
int moeq_nvfp4_to_mxfp4_device(const uint8_t* nib, const uint8_t* e4m3, const float* scale2, int rows, int cols, int n,
                               uint8_t* nib_out, uint8_t* e8m0_out, uint32_t* status, void* stream);

/* ------------------------------------------------------------------ kernels */

/* Dequantise expert `expert` of w to fp32 [rows][cols]. The value is the format's
 * exact weight rounded once to fp32 (exact for MXFP4, IQ2_XXS, FP8_B128). */
int moeq_dequant(const moeq_weight* w, int expert, float* out, void* stream);

/* Workspace bytes needed by moeq_expert_forward / the stage entry points for T
 * tokens. The workspace must be zero-filled once before first use (or passed to
 * moeq_workspace_init); its first 4 bytes hold the sticky device error word. */
size_t moeq_workspace_bytes(const moeq_layer* L, int T);
int moeq_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* y[T][H] (fp32, overwritten) of the routed layer for x[T][H] (bf16), expert ids
 * ids[T][K] (int32) and route weights rw[T][K] (fp32, applied after down as given).
 * Decode path (any format: the stage kernels below) below T = 128 tokens. From
 * T = 128, each MXFP4 projection that meets the prefill stages' shape and
 * alignment conditions (below) runs the W4A8 prefill GEMM instead (gate/up on x
 * quantised to MXFP8; down on h quantised to MXFP8), whatever the format of the
 * other projection: a layer mixing IQ2_XXS (or Q2_K) and MXFP4 projections takes
 * the W4A8 GEMM for its MXFP4 projection and the grouped decode kernels for the
 * other (1x Spark forum thread, second post: one grouped GEMM per projection).
 * T == 0 is a no-op. x, y 16-byte aligned. */
int moeq_expert_forward(const moeq_layer* L, const void* x, const int32_t* ids, const float* rw, int T, float* y,
                        void* ws, size_t ws_bytes, void* stream);

/* moeq_expert_forward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). It runs the same kernels on the same path,
 * with their scratch (routing, h, partials, MXFP8 buffers) in a fixed device
 * array inside the library: MOEQ_NOALLOC_SCRATCH_BYTES per GPU, held until the
 * process ends, its address taken once per device on the first call. No call
 * allocates or frees anything. A call whose moeq_workspace_bytes(L, T) exceeds
 * the scratch returns MOEQ_E_SCRATCH before any launch (at hidden 4096,
 * intermediate 2048, 256 experts, top-6: up to T = 227 tokens on the decode path;
 * an all-MXFP4 layer takes the prefill path from T = 128, up to T = 204). Every call on a GPU shares that GPU's scratch: calls
 * that overlap on one GPU (two streams, or two threads) race and must be
 * serialised by the caller; nothing in the scratch has to start at zero.
 * dev_err (device memory, 4-byte aligned, may be NULL) receives the
 * MOEQ_DEVERR_* bits by OR; with NULL they go to a word nobody reads. Other
 * arguments, checks and outputs as moeq_expert_forward. */
#define MOEQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int moeq_expert_forward_noalloc(const moeq_layer* L, const void* x, const int32_t* ids, const float* rw, int T,
                                float* y, uint32_t* dev_err, void* stream);

/* Stages of the decode path, for tests and timing (moeq_expert_forward runs them
 * in order). moeq_route groups the T*K (token, slot) pairs by expert into the
 * workspace (needed before the other two when T > 1). moeq_gate_up writes
 * h[T][K][I] (fp32) = silu(G x) * (U x) per pair. moeq_down writes y[T][H].
 * x, h, y 16-byte aligned. */
int moeq_route(const moeq_layer* L, const int32_t* ids, int T, void* ws, size_t ws_bytes, void* stream);
int moeq_gate_up(const moeq_layer* L, const void* x, const int32_t* ids, int T, float* h, void* ws, size_t ws_bytes,
                 void* stream);
int moeq_down(const moeq_layer* L, const float* h, const int32_t* ids, const float* rw, int T, float* y, void* ws,
              size_t ws_bytes, void* stream);

/* moeq_gate_up with its kernel launched so that start_event / stop_event (two
 * hipEvent_t created with timing, passed as void*) record the kernel's own start
 * and end, for timing that excludes queue gaps. Same arguments and outputs. */
int moeq_gate_up_timed(const moeq_layer* L, const void* x, const int32_t* ids, int T, float* h, void* ws,
                       size_t ws_bytes, void* stream, void* start_event, void* stop_event);

/* Stages of the W4A8 prefill path, one per projection (its weights MXFP4, else
 * MOEQ_E_FMT; the other projection may be in any format; hidden and inter
 * multiples of 256; the stage's weight scale planes and their expert stride
 * 8-byte aligned, else MOEQ_E_ALIGN; moeq_route first, on the same workspace).
 * moeq_prefill_gate_up: xq/xs = MXFP8 x (codes u8 [T][H], 16-byte aligned; e8m0
 *   u8 [T][H/32], 8-byte aligned) -> hq/hs = MXFP8 h (codes u8 [T*K][I], e8m0 u8
 *   [T*K][I/32]); h_f32 (may be NULL) receives h before quantisation, fp32 [T*K][I].
 * moeq_prefill_down: hq/hs (same alignment as xq/xs) -> y[T][H] (16-byte
 *   aligned); T >= 2.
 * MOEQ_E_FMT for other formats, MOEQ_E_SHAPE for other shapes. */
int moeq_prefill_gate_up(const moeq_layer* L, const uint8_t* xq, const uint8_t* xs, const int32_t* ids, int T,
                         float* h_f32, uint8_t* hq, uint8_t* hs, void* ws, size_t ws_bytes, void* stream);
int moeq_prefill_down(const moeq_layer* L, const uint8_t* hq, const uint8_t* hs, const int32_t* ids, const float* rw,
                      int T, float* y, void* ws, size_t ws_bytes, void* stream);

/* Dense block-quantized linear y[T][rows] = W_expert x[T][cols] (fp32 out). Any
 * format; FP8_B128 is the dense-layer format (IQ2_XXS + Q2_K + FP8 hybrid card).
 * MXFP8, MXFP8_TILED and FP8_B32 run on the block-scaled FP8 matrix instruction
 * for every T (the weights' e8m0 scale is the instruction's scale; x enters as
 * two E4M3 terms per value with e8m0 scales per 32, exact to 2^-21.8 of each
 * 32-block's maximum): rows a multiple of 16 (FP8_B32: 32), cols a multiple of
 * 128 (MXFP8_TILED: 512) and at most 8192, else MOEQ_E_SHAPE.
 * x bf16 [T][cols], 16-byte aligned; y fp32 [T][rows], 4-byte aligned; both
 * caller-owned, y overwritten. FP8_B128 with T >= 2 and cols a multiple of 256
 * runs on the bf16 matrix instruction (E4M3 codes exact in bf16, block scale
 * applied to each 128-wide K tile's fp32 partial); otherwise one GEMV pass per
 * token group, which needs cols / (weights per 16-byte chunk) <= 256 (MOEQ_E_SHAPE
 * beyond). Asynchronous on `stream`. */
int moeq_linear(const moeq_weight* w, int expert, const void* x, int T, float* y, void* stream);

/* MXFP8 quantisation of rows of K values (K a multiple of 32): per 32 consecutive
 * values, e8m0 code E = clamp(e + 127, 0, 254) with 2^e the smallest power of two
 * keeping max|v| / 2^e <= 448 (e = p-9 if the frexp mantissa of max|v| is <= 0.875,
 * else p-8; all-zero block: E = 0, codes 0); codes = E4M3FN round-to-nearest-even of
 * v / 2^(E-127), saturating, sign kept (1x Spark forum thread, second post: E4M3
 * activations with a dynamic scale; the 32-wide block and the non-clipping scale
 * rule are this library's reading). moeq_quantize_mxfp8 takes bf16 input x [T][K]
 * (the prefill activations), moeq_quantize_mxfp8_f32 fp32 (the intermediate h).
 * x and q 16-byte aligned, caller-owned device memory; q u8 [T][K] and e8m0 u8
 * [T][K/32] overwritten. MOEQ_E_SHAPE if K is not a positive multiple of 32. */
int moeq_quantize_mxfp8(const void* x, int T, int K, uint8_t* q, uint8_t* e8m0, void* stream);
int moeq_quantize_mxfp8_f32(const float* x, int T, int K, uint8_t* q, uint8_t* e8m0, void* stream);

/* Synchronise `stream`, then read (and with clear != 0, zero) the device error word. */
int moeq_check_device_error(void* ws, void* stream, uint32_t* err_host, int clear);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ_H_ */
