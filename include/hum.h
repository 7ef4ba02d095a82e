/*
 * hum.h -- C ABI of the MI355X (gfx950) quantized GEMM library.
 *
 * One quantization description (weight format, scale granularity, scale
 * dtype, zero point, second-level scale, activation format) drives weight
 * preparation and the dense / MoE GEMMs.  The description follows "Announcing
 * Humming: Fast, Flexible Kernels for Quantized Inference", section "Unified
 * quantization representation"; the preparation step (validate, pad, repack
 * into the kernel layout) follows section "Per-workload tuning and JIT
 * compilation" of the same post.
 *
 * Conventions for every entry point:
 *  - Memory: every pointer argument that names tensor data is a DEVICE
 *    pointer owned by the caller (the library allocates nothing).  Host
 *    pointers are only the descriptor / config structs.
 *  - Streams: work is enqueued on `stream` (a hipStream_t passed as void*;
 *    NULL means the default stream) and is ordered with the caller's other
 *    work on that stream.  No entry point synchronizes the device.
 *  - Errors: argument / shape / format errors return a non-zero hum_status
 *    before anything is launched; hum_last_error() then describes the
 *    problem (thread-local string).  A failed launch returns HUM_ERR_HIP.
 *  - Layout: row-major, K contiguous.  4-bit codes are packed two per byte,
 *    the even k in the low nibble.
 *  - Limits: K must be a multiple of 128; N is arbitrary.  Integer (INT4 /
 *    UINT4) group sizes must be multiples of 128; MXFP4 uses group 32 with
 *    E8M0 scales.
 */
#ifndef HUM_H_
#define HUM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hum_status {
  HUM_OK = 0,
  HUM_ERR_INVALID_ARG = 1,  /* NULL pointer, bad size, inconsistent shapes */
  HUM_ERR_UNSUPPORTED = 2,  /* valid description this library does not run */
  HUM_ERR_WORKSPACE = 3,    /* buffer smaller than the matching *_bytes() query */
  HUM_ERR_HIP = 4           /* a HIP launch / runtime call failed */
} hum_status;

typedef enum hum_dtype {
  HUM_BF16 = 0,
  HUM_F32 = 1,
  HUM_INT4 = 2,   /* signed two's-complement nibble, -8..7; with HUM_E8M0
                     scales per 32 along K: MXINT4 (bf16 activations) */
  HUM_UINT4 = 3,  /* unsigned nibble 0..15, optional zero point */
  HUM_E2M1 = 4,   /* FP4 (MXFP4 element) */
  HUM_E4M3 = 5,   /* FP8 E4M3 "FN": max 448, NaN = 0x7F/0xFF, no Inf; as a
                     scale dtype: NVFP4's group scale (E2M1 weights, G = 16,
                     finite codes) */
  HUM_E8M0 = 6,   /* power-of-two scale 2^(c-127) */
  HUM_INT8 = 7,   /* signed two's-complement byte, -128..127 (W8A16: bf16
                     activations, per-channel or per-tensor f32 scales) */
  /* Low-bit integer weights ("Announcing Humming", section "WnA16": the
     shared dequantization path covers INT1, INT2 and INT3 as well): b-bit
     codes packed as an LSB-first bit stream along K (code k of a row at
     bits b*k .. b*k+b-1 of the row's bytes read as one little-endian
     integer; codes [E][N][K*b/8]).  Signed: two's complement; unsigned:
     0..2^b-1 with an optional zero point.  bf16 activations, bf16 / f32
     scales per tensor, channel or group (G a multiple of 128). */
  HUM_INT3 = 8,   /* -4..3 */
  HUM_UINT3 = 9,  /* 0..7 */
  HUM_INT2 = 10,  /* -2..1 */
  HUM_UINT2 = 11, /* 0..3 */
  HUM_INT1 = 12,  /* -1..0 */
  HUM_UINT1 = 13, /* 0..1 */
  /* FP6 weights (OCP MX v1.0 element types; "WnA16" in the Humming
     announcement runs FP4 to FP8 weights): codes packed as an LSB-first 6-bit
     stream along K ([E][N][K*6/8]), an E8M0 scale per 32 along K (MXFP6),
     bf16 activations. */
  HUM_E2M3 = 14,  /* exponent bias 1, 3 mantissa bits, max 7.5 */
  HUM_E3M2 = 15   /* exponent bias 3, 2 mantissa bits, max 28 */
} hum_dtype;

typedef enum hum_scale_gran {
  HUM_SCALE_TENSOR = 0,   /* one scale per expert          : scales [E][1][1] */
  HUM_SCALE_CHANNEL = 1,  /* one scale per output channel  : scales [E][N][1] */
  HUM_SCALE_GROUP = 2,    /* one scale per group along K   : scales [E][N][K/G] */
  HUM_SCALE_BLOCK = 3     /* one scale per G x G block of W (rows n, columns k):
                             scales [E][ceil(N/G)][K/G]; E4M3 weights, G = 128
                             (block-scaled FP8 W8A8) */
} hum_scale_gran;

typedef enum hum_act_fmt {
  HUM_ACT_BF16 = 0,       /* bf16 activations as given (WnA16) */
  HUM_ACT_FP8_TOKEN = 1,  /* E4M3 codes + one f32 scale per row (W8A8) */
  HUM_ACT_MXFP8 = 2,      /* E4M3 codes + one E8M0 scale per 32 along K (W4A8) */
  HUM_ACT_MXFP4 = 3,      /* E2M1 codes, two per byte (even k in the low nibble),
                             + one E8M0 scale per 32 along K (W4A4) */
  HUM_ACT_FP8_GROUP = 4   /* E4M3 codes + one f32 scale per row per 128 along K
                             (block-scaled FP8 W8A8, dense only) */
} hum_act_fmt;

/* The quantization description of one weight tensor [E][N][K]. */
typedef struct hum_weight_desc {
  int32_t weight_dtype;      /* HUM_INT4 | HUM_UINT4 | HUM_INT8 | HUM_E2M1 | HUM_E4M3 |
                                HUM_INT3 .. HUM_UINT1 */
  int32_t scale_gran;        /* hum_scale_gran */
  int32_t group_size;        /* K elements per group (HUM_SCALE_GROUP), block edge (HUM_SCALE_BLOCK) */
  int32_t scale_dtype;       /* HUM_BF16 | HUM_F32 | HUM_E8M0 */
  int32_t has_zero_point;    /* 0/1; unsigned integer codes only (UINT4 .. UINT1);
                                zeros u8 [E][N][K/G] (0..2^b-1) */
  int32_t has_global_scale;  /* 0/1; second-level f32 scale per expert, [E] */
  int32_t act_fmt;           /* hum_act_fmt the layer runs with */
  int32_t num_experts;       /* E >= 1 (dense layers use 1) */
  int64_t n;                 /* output channels per expert */
  int64_t k;                 /* reduction length */
} hum_weight_desc;

typedef enum hum_kernel_kind {
  HUM_KERNEL_TILE = 0,    /* prefill: 4 waves along N share an LDS activation tile */
  HUM_KERNEL_STREAM = 1,  /* decode: one 16-row tile, waves_k waves stream K */
  HUM_KERNEL_TILE32 = 2   /* prefill with 32 x 32 MFMA blocks (bf16 activations,
                             INT / MXFP4 weights; wave_m, wave_n even) */
} hum_kernel_kind;

/* Tile / split-K configuration (output of the selector, or forced). */
typedef struct hum_tile_config {
  int32_t kind;      /* hum_kernel_kind */
  int32_t wave_m;    /* 16-row MFMA sub-tiles per wave (rows per WG = 16*wave_m) */
  int32_t wave_n;    /* 16-column sub-tiles per wave */
  int32_t waves_n;   /* waves of a workgroup side by side along N */
  int32_t waves_k;   /* waves of a workgroup splitting K (in-WG split-K) */
  int32_t split_k;   /* workgroups splitting K (fp32 partials + reduce kernel) */
  int32_t block_m;   /* rows per workgroup tile = MoE expert block (16*wave_m) */
  int32_t stages;    /* tile kernel: K-blocks of operands staged in LDS at once
                        (2 or 3; 0 = 2); ignored by the stream kernel */
  int32_t stream_k;  /* dense tile kernels: 0 = off; G > 0 = Stream-K ("Device-
                        specific tuning" in the Humming announcement lists it
                        among the task mappings): G workgroups share the tiles'
                        K-blocks evenly, a tile shared by several is summed by
                        the last of them to finish, in a fixed order (fp32
                        partials; split_k must be 1; at most 16384 tiles) */
} hum_tile_config;

/* ---- weight preparation ------------------------------------------------ */

/* Bytes of the packed (kernel-layout) buffer for `desc`; 0 if the
 * description is invalid or unsupported (see hum_last_error()). */
size_t hum_packed_weight_bytes(const hum_weight_desc* desc);

/* Canonical ("standard format") tensors -> packed kernel layout.
 *   codes  : u8 [E][N][K/2] (4-bit), [E][N][K] (INT8, E4M3) or
 *            [E][N][K*b/8] (b-bit integers, b = 1, 2, 3; FP6: b = 6)
 *   scales : [E][N'][K/G'] in scale_dtype (N' = 1 for TENSOR, G' per gran)
 *   zeros  : u8 [E][N'][K/G'] or NULL when has_zero_point == 0
 *   global_scale : f32 [E] or NULL when has_global_scale == 0
 *   packed : device buffer of at least hum_packed_weight_bytes(desc)
 * Pads N to a multiple of 16 with codes that decode to zero and converts
 * group size K (and per-tensor scales) to the per-channel form. */
hum_status hum_prepare_weight(const hum_weight_desc* desc, const void* codes,
                              const void* scales, const void* zeros,
                              const float* global_scale, void* packed,
                              size_t packed_bytes, void* stream);

/* Test export: packed -> f32 [E][N][K] of (v(q) - z) * S, excluding the
 * second-level scale.  Exact for every supported format. */
hum_status hum_dequant_weight(const hum_weight_desc* desc, const void* packed,
                              float* out, void* stream);

/* ---- activation quantizer ---------------------------------------------- */

/* bf16 x [m][k] (row stride ld_x elements) -> E4M3 codes q [m][k] plus
 *   HUM_ACT_FP8_TOKEN : scales f32 [m], s = amax/448 (1 for a zero row),
 *                       q = E4M3_RNE_SAT(x / s) with an IEEE f32 division;
 *   HUM_ACT_MXFP8     : scales u8 [m][k/32], E = clamp(floor(log2 amax) - 8
 *                       + 127, 0, 254) (127 for a zero block),
 *                       q = E4M3_RNE_SAT(x / 2^(E-127));
 *   HUM_ACT_FP8_GROUP : scales f32 [m][k/128], the FP8_TOKEN rule applied to
 *                       each group of 128 along k;
 *   HUM_ACT_MXFP4     : E2M1 codes q [m][k/2] (two per byte, even k in the
 *                       low nibble), scales u8 [m][k/32], E = clamp(floor(
 *                       log2 amax) - 2 + 127, 0, 254) (127 for a zero block),
 *                       q = E2M1_RNE_SAT(x / 2^(E-127)) (saturated to +-6).
 * The formats are those named in the "End-to-end inference performance"
 * ("tokenwise FP8"), "Choosing the activation type" (MXFP8) and "W8A8 /
 * W4A8 / W4A4" (MXFP4 activations) sections of the Humming announcement;
 * the scale rules are the OCP ones (FP8_GROUP: the activations of the
 * block-scaled FP8 W8A8 of the same section).  k must be a multiple of 32
 * for MXFP8 and MXFP4, of 128 for FP8_GROUP. */
hum_status hum_quant_act(int32_t act_fmt, int64_t m, int64_t k, const void* x_bf16,
                         int64_t ld_x, void* q, void* scales, void* stream);

/* ---- dense layer --------------------------------------------------------- */

/* Workspace bytes hum_linear needs for m rows (quantized activations,
 * row sums, split-K partials). */
size_t hum_linear_workspace_bytes(const hum_weight_desc* desc, int64_t m);

/* C[m][n] = A[m][:] . W[n][:] (+ bias[n]) -> bf16, fp32 accumulation
 * ("WnA16" and "W8A8 / W4A8 / W4A4" sections of the Humming announcement).
 *   a        : bf16 [m][k]; or, when act_fmt != BF16 and a_scales != NULL,
 *              already-quantized codes with their scales, as hum_quant_act
 *              writes them: E4M3 [m][k] + f32 [m] (FP8_TOKEN), E4M3 [m][k] +
 *              E8M0 u8 [m][k/32] (MXFP8), E2M1 pairs u8 [m][k/2] + E8M0 u8
 *              [m][k/32] (MXFP4), E4M3 [m][k] + f32 [m][k/128] (FP8_GROUP)
 *   bias     : bf16 [n] or NULL
 *   out      : bf16 [m][n] (row stride n)
 *   workspace: device buffer of hum_linear_workspace_bytes(desc, m) bytes
 *              (quantized activations, row sums, split-K partials); its
 *              contents need no initialisation.  Calls that overlap in time
 *              must use different workspaces.
 * Only num_experts == 1 descriptions are dense layers. */
hum_status hum_linear(const hum_weight_desc* desc, const void* packed, int64_t m,
                      const void* a, const void* a_scales, const void* bias,
                      void* out, void* workspace, size_t ws_bytes, void* stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): hum_linear with no
 * workspace argument.  The workspace (split-K partials, activations
 * quantized in the call, row sums) lives in a static device array of
 * HUM_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until
 * the process ends; no entry point allocates.  The selector's configuration
 * is used; a call whose workspace would exceed the array is refused with
 * HUM_ERR_WORKSPACE before anything is launched.  The array's contents need
 * no initialisation and are left as the last call wrote them.  Calls on one
 * GPU share the array: calls that overlap in time (different streams) race,
 * so one stream (or ordered streams) per GPU.  Arguments as hum_linear. */
#define HUM_NOALLOC_SCRATCH_BYTES (32u << 20)
hum_status hum_linear_noalloc(const hum_weight_desc* desc, const void* packed, int64_t m,
                              const void* a, const void* a_scales, const void* bias,
                              void* out, void* stream);

/* hum_linear with an explicit tile configuration (NULL = selector).  On the
 * decode kernel (kind HUM_KERNEL_STREAM) a W4A4 description runs as E4M3 x
 * E2M1 and quantizes its bf16 activations itself (each MXFP4 code as the
 * E4M3 byte of its value), and a block-scaled FP8 description quantizes its
 * bf16 rows itself (per row and 128 along K); pre-quantized activations
 * with such a configuration are refused (HUM_ERR_UNSUPPORTED), and the
 * selector gives them a tile configuration. */
hum_status hum_linear_ex(const hum_weight_desc* desc, const void* packed, int64_t m,
                         const void* a, const void* a_scales, const void* bias,
                         void* out, void* workspace, size_t ws_bytes,
                         const hum_tile_config* cfg, void* stream);

/* Workspace bytes hum_linear_ex needs with configuration `cfg`
 * (NULL = the selector's choice). */
size_t hum_linear_workspace_bytes_ex(const hum_weight_desc* desc, int64_t m,
                                     const hum_tile_config* cfg);

/* Zero a device buffer (enqueued on `stream`; a fill kernel, so it can be
 * captured in a HIP graph).
 * Workspaces: the first HUM_WS_HEADER_BYTES of every workspace hold the
 * Stream-K tile counters, which must be zero before the workspace's first
 * call (this call, once) and which every call leaves zero; the rest needs
 * no initialisation.  Calls that may overlap in time need different
 * workspaces. */
#define HUM_WS_HEADER_BYTES (64u << 10)
hum_status hum_prepare_workspace(void* workspace, size_t ws_bytes, void* stream);

/* Selector: the tile / split-K configuration hum_linear would use for m
 * rows (pure host function of the description, m and the device).  Device
 * heuristics per M range follow "Device-parameter tuning" in the Humming
 * announcement. */
hum_status hum_select_config(const hum_weight_desc* desc, int64_t m,
                             hum_tile_config* cfg_out);

/* Selection flags. */
#define HUM_SELECT_BATCH_INVARIANT 1u  /* every output row independent of m and
                                          of the other rows of the call */
#define HUM_SELECT_MOE_GATE_UP 2u      /* hum_moe_select_config: the gate_up
                                          GEMM's configuration (default: the
                                          down GEMM's) */

/* hum_select_config with flags ("batch invariance" among the compute options
 * in the Humming announcement's feature list).  HUM_SELECT_BATCH_INVARIANT
 * returns a tile-kernel configuration without split-K: the tile kernel sums
 * each row in one fixed order for every tile shape, so a row's bf16 output is
 * bitwise the same for any m when hum_linear_ex runs with the configuration
 * this returns for that m.  Other flag bits are an error (HUM_ERR_INVALID_ARG). */
hum_status hum_select_config_ex(const hum_weight_desc* desc, int64_t m, uint32_t flags,
                                hum_tile_config* cfg_out);

/* On-device autotune ("Autotune" under future work in the Humming
 * announcement): times every compiled dense configuration that fits
 * `ws_bytes` (with HUM_SELECT_BATCH_INVARIANT, only the batch-invariant ones)
 * on the caller's buffers -- one untimed call, then `iters` calls between
 * two HIP events on `stream` -- and returns the fastest in *best_out and its
 * mean time per call in µs in *best_us_out (may be NULL).  The arguments
 * are those of hum_linear_ex; `out` ends holding the winner's result.
 * Blocks the host until the timing completes: not for graph capture.
 * Callers cache the result per (description, m).  HUM_ERR_UNSUPPORTED when
 * no configuration fits the workspace. */
hum_status hum_autotune_linear(const hum_weight_desc* desc, const void* packed, int64_t m,
                               const void* a, const void* a_scales, const void* bias,
                               void* out, void* workspace, size_t ws_bytes, int32_t iters,
                               uint32_t flags, hum_tile_config* best_out, float* best_us_out,
                               void* stream);

/* ---- MoE layer ----------------------------------------------------------- */

/* Workspace bytes hum_moe_gemm needs for T tokens routed to topk experts. */
size_t hum_moe_workspace_bytes(const hum_weight_desc* w13, const hum_weight_desc* w2,
                               int64_t num_tokens, int32_t topk);

/* Full MoE expert layer ("indexed" grouping: rows gathered through the
 * sorted routing ids; SGLang PR #23754 summary, "Key source snippets").
 * Expert formats: MXFP4 (bf16, MXFP8 or MXFP4 activations), MXINT4 and
 * NVFP4 (bf16), E4M3 per-channel / per-tensor (bf16 or per-token FP8
 * activations), E4M3 with 128 x 128 block scales (per-group FP8) and INT8
 * (bf16); w13 and w2 share one format.  FP8 activation formats quantize
 * the bf16 SwiGLU output with the same rule before the down GEMM:
 *   align (sort token slots by expert) -> gate_up grouped GEMM with a fused
 *   SwiGLU (a = silu(h[:I]) * h[I:], requantized to MXFP8 for W4A8) -> down
 *   grouped GEMM -> top-k weighted reduce.
 *   w13 : [E][2I][H] description + packed buffer; w2 : [E][H][I]
 *   x   : bf16 [T][H]; topk_ids i32 [T][topk]; topk_weights f32 [T][topk]
 *   out : bf16 [T][H]
 * A slot whose id lies outside [0, E) (for example -1 for an expert held
 * on another device) is skipped: it adds nothing to out.  At most 512
 * experts.
 * No device->host synchronization: grids are sized from T, topk and E. */
hum_status hum_moe_gemm(const hum_weight_desc* w13, const void* packed_w13,
                        const hum_weight_desc* w2, const void* packed_w2,
                        int64_t num_tokens, int32_t topk, const void* x_bf16,
                        const int32_t* topk_ids, const float* topk_weights,
                        void* out_bf16, void* workspace, size_t ws_bytes, void* stream);

/* hum_moe_gemm with an explicit configuration (NULL = selector); the gate_up
 * and down GEMMs share cfg's tile shape and block_m = 16 * cfg->wave_m
 * (wave_n must be a multiple of 4 for the MXFP8 SwiGLU epilogue). */
hum_status hum_moe_gemm_ex(const hum_weight_desc* w13, const void* packed_w13,
                           const hum_weight_desc* w2, const void* packed_w2,
                           int64_t num_tokens, int32_t topk, const void* x_bf16,
                           const int32_t* topk_ids, const float* topk_weights,
                           void* out_bf16, void* workspace, size_t ws_bytes,
                           const hum_tile_config* cfg, void* stream);

/* The configuration for hum_moe_gemm_ex (both GEMMs) at T tokens.  flags = 0:
 * the selector's down-GEMM configuration (hum_moe_gemm itself may run a small
 * batch's gate_up GEMM on the decode kernel); HUM_SELECT_MOE_GATE_UP: the
 * gate_up GEMM's.  HUM_SELECT_BATCH_INVARIANT: a tile-kernel configuration,
 * with which every token's output row is bitwise independent of T and of the
 * other tokens' routing. */
hum_status hum_moe_select_config(const hum_weight_desc* w13, const hum_weight_desc* w2,
                                 int64_t num_tokens, int32_t topk, uint32_t flags,
                                 hum_tile_config* cfg_out);

/* On-device autotune of the MoE layer, as hum_autotune_linear does for dense
 * ones: every compiled configuration (both GEMMs share it, no split-K; with
 * HUM_SELECT_BATCH_INVARIANT tile kernels only) whose workspace fits
 * `ws_bytes` is run once untimed and `iters` times between HIP events on the
 * caller's buffers; the fastest is returned with its mean µs per layer call,
 * and `out_bf16` ends holding its result.  The arguments are those of
 * hum_moe_gemm_ex.  Blocks the host; not for graph capture. */
hum_status hum_autotune_moe(const hum_weight_desc* w13, const void* packed_w13,
                            const hum_weight_desc* w2, const void* packed_w2,
                            int64_t num_tokens, int32_t topk, const void* x_bf16,
                            const int32_t* topk_ids, const float* topk_weights,
                            void* out_bf16, void* workspace, size_t ws_bytes, int32_t iters,
                            uint32_t flags, hum_tile_config* best_out, float* best_us_out,
                            void* stream);

/* Workspace bytes hum_moe_gemm_ex needs with configuration `cfg`. */
size_t hum_moe_workspace_bytes_ex(const hum_weight_desc* w13, const hum_weight_desc* w2,
                                  int64_t num_tokens, int32_t topk,
                                  const hum_tile_config* cfg);

/* The expert layer on the "grouped_masked" layout (the EP low-latency
 * receive format; a gemm_type of the MoE runner in the SGLang PR #23754
 * summary, "Key source snippets"): expert e's rows are
 * x[e][0 : expert_num_tokens[e]] of a bf16 [E][max_m][H] buffer, and
 *   out[e][i] = down(SwiGLU(gate_up(x[e][i])))   for i < expert_num_tokens[e]
 * in bf16 [E][max_m][H], with no top-k weighting (the combine after the
 * layer applies it).  Rows i >= expert_num_tokens[e] of out are not written.
 *   expert_num_tokens : i32 [E] on the device, each clamped to [0, max_m];
 *                       read by the kernels only (no device->host copy)
 *   max_m             : rows per expert buffer, a multiple of 16
 *   expected_m        : the caller's host-side estimate of rows per expert;
 *                       it picks the tile (the expert block must divide max_m)
 *   cfg               : NULL = selector, else both GEMMs' configuration
 * Same weight formats and activation formats as hum_moe_gemm; rows of x past
 * an expert's count are read (quantized) but never reach out. */
hum_status hum_moe_gemm_masked(const hum_weight_desc* w13, const void* packed_w13,
                               const hum_weight_desc* w2, const void* packed_w2,
                               int64_t max_m, int64_t expected_m, const void* x_bf16,
                               const int32_t* expert_num_tokens, void* out_bf16,
                               void* workspace, size_t ws_bytes,
                               const hum_tile_config* cfg, void* stream);

/* Workspace bytes hum_moe_gemm_masked needs (0 on invalid arguments). */
size_t hum_moe_masked_workspace_bytes(const hum_weight_desc* w13, const hum_weight_desc* w2,
                                      int64_t max_m, int64_t expected_m,
                                      const hum_tile_config* cfg);

/* Stage export: sort the flat routing slots f = t*topk + j by expert.
 *   sorted  : i32 [T*topk + E*(block_m-1)]; segment of expert e starts at
 *             offsets[e], holds its slots in ascending f, is padded to a
 *             multiple of block_m with the sentinel T*topk (as is the tail)
 *   offsets : i32 [E+1]; counts : i32 [E]
 * ("moe_align_block_size" / "moe_permute_prepare" in the SGLang PR #23754
 * summary, "Implementation breakdown" and "Review highlights"). */
hum_status hum_moe_align(const int32_t* topk_ids, int64_t num_tokens, int32_t topk,
                         int32_t num_experts, int32_t block_m, int32_t* sorted,
                         int32_t* offsets, int32_t* counts, void* stream);

/* The same sort with scratch for large routing tables, which many
 * workgroups then share (the result is identical).  workspace: device
 * buffer of hum_moe_align_workspace_bytes(num_tokens, topk, num_experts)
 * bytes (0 when the table is small enough for one workgroup; NULL is then
 * accepted); HUM_ERR_WORKSPACE if smaller. */
size_t hum_moe_align_workspace_bytes(int64_t num_tokens, int32_t topk, int32_t num_experts);
hum_status hum_moe_align_ex(const int32_t* topk_ids, int64_t num_tokens, int32_t topk,
                            int32_t num_experts, int32_t block_m, int32_t* sorted,
                            int32_t* offsets, int32_t* counts, void* workspace,
                            size_t ws_bytes, void* stream);

/* Stage export: out[t] = bf16(sum_j w[t][j] * y[t*topk + j]) with y bf16
 * [T*topk][h] indexed by flat slot, fp32 sum in fixed j order
 * ("moe_fused_mul_sum" in the SGLang PR #23754 summary). */
hum_status hum_moe_reduce(const void* y_bf16, const float* topk_weights,
                          int64_t num_tokens, int32_t topk, int64_t h,
                          void* out_bf16, void* stream);

/* Stage export: one grouped GEMM of a MoE layer over rows sorted by expert
 * (the per-gemm_type runner paths of the SGLang PR #23754 summary, "Key
 * source snippets"; the "Gateup" and "Down" GEMMs of the Humming
 * announcement's "Performance" section), with the sorted order and padded
 * offsets that hum_moe_align returns.
 *   w, packed   : expert weights [E][N][K] (the formats hum_moe_gemm runs)
 *   a_mode      : HUM_MOE_A_GATHER : sorted row r reads a[sorted[r] / topk]
 *                                    (a: [num_tokens][K], the layer input)
 *                 HUM_MOE_A_SORTED : sorted row r reads a[r]
 *                                    (a: [sorted_len][K], e.g. the SwiGLU
 *                                    output of the gate_up stage)
 *   a, a_scales : activations in w's activation format: bf16, or codes and
 *                 scales as hum_quant_act writes them (this call quantizes
 *                 nothing)
 *   sorted      : i32 [sorted_len], sentinel num_tokens * topk for padding
 *   offsets     : i32 [E + 1], padded to block_m (block_m = 16, 32, 64, 128)
 *   epilogue    : HUM_MOE_EPI_NONE         bf16 out [sorted_len][N]
 *                 HUM_MOE_EPI_SCATTER      bf16 out [num_tokens*topk][N] at
 *                                          row sorted[r] (flat slot order)
 *                 HUM_MOE_EPI_SWIGLU_BF16  bf16 out [sorted_len][N/2] of
 *                                          silu(h[:N/2]) * h[N/2:]
 *                 HUM_MOE_EPI_SWIGLU_MXFP8 E4M3 out [sorted_len][N/2] + E8M0
 *                                          out_scales [sorted_len][N/64]
 *                 HUM_MOE_EPI_SWIGLU_MXFP4 E2M1 pairs out [sorted_len][N/4] +
 *                                          E8M0 out_scales [sorted_len][N/64]
 *                 (the SwiGLU epilogue must be the activation format's: MX
 *                 requantization for MXFP8 / MXFP4, bf16 otherwise)
 *   out_swiglu_f32 : optional f32 [sorted_len][N/2]: the SwiGLU values the
 *                 epilogue rounded or requantized
 *   cfg         : NULL = a configuration with block_m-row tiles
 *   workspace   : hum_moe_grouped_gemm_workspace_bytes(...) bytes
 * Padding rows (sorted[r] >= num_tokens * topk) are never stored. */
typedef enum hum_moe_a_mode { HUM_MOE_A_GATHER = 0, HUM_MOE_A_SORTED = 1 } hum_moe_a_mode;
typedef enum hum_moe_epilogue {
  HUM_MOE_EPI_NONE = 0,
  HUM_MOE_EPI_SCATTER = 1,
  HUM_MOE_EPI_SWIGLU_BF16 = 2,
  HUM_MOE_EPI_SWIGLU_MXFP8 = 3,
  HUM_MOE_EPI_SWIGLU_MXFP4 = 4
} hum_moe_epilogue;

size_t hum_moe_grouped_gemm_workspace_bytes(const hum_weight_desc* w, int32_t a_mode, int32_t epilogue,
                                            int64_t num_tokens, int32_t topk, int64_t sorted_len,
                                            int32_t block_m, const hum_tile_config* cfg);

hum_status hum_moe_grouped_gemm(const hum_weight_desc* w, const void* packed, int32_t a_mode,
                                int32_t epilogue, int64_t num_tokens, int32_t topk, const void* a,
                                const void* a_scales, const int32_t* sorted, int64_t sorted_len,
                                const int32_t* offsets, int32_t block_m, void* out, void* out_scales,
                                float* out_swiglu_f32, const hum_tile_config* cfg, void* workspace,
                                size_t ws_bytes, void* stream);

/* ---- measurement -------------------------------------------------------- */

/* Device peak probes (measurement only; the GEMM path never calls them).
 * Enqueue on `stream` one launch of a probe kernel and report its work in
 * *work_out (bytes read, or flops), to be timed by the caller:
 *   HUM_PEAK_HBM_READ     : stream-read n bytes of the device buffer buf
 *                           (n a multiple of 16)
 *   HUM_PEAK_MFMA_*       : n iterations of eight independent matrix
 *                           instructions per wave on every CU (bf16
 *                           16x16x32; E4M3 x E4M3, E2M1 x E2M1 and E4M3 x
 *                           E2M1 16x16x128)
 *   HUM_PEAK_MFMA32_*     : the same rates with the 32x32 shapes (four
 *                           independent instructions per wave)
 *   sink : device buffer of at least 2048 * 256 * 4 bytes (probe results
 *          land there so that no work is dead).
 * The rooflines the bench reports against are the published MI355X peaks;
 * these re-measure what the box sustains. */
#define HUM_PEAK_HBM_READ 0
#define HUM_PEAK_MFMA_BF16 1
#define HUM_PEAK_MFMA_FP8 2
#define HUM_PEAK_MFMA_FP4 3
#define HUM_PEAK_MFMA_FP8_FP4 4
#define HUM_PEAK_MFMA32_BF16 5     /* the 32x32 shapes: bf16 32x32x16, f8f6f4 32x32x64 */
#define HUM_PEAK_MFMA32_FP8 6
#define HUM_PEAK_MFMA32_FP4 7
#define HUM_PEAK_MFMA32_FP8_FP4 8
hum_status hum_peak_probe(int32_t kind, int64_t n, const void* buf, void* sink, double* work_out,
                          void* stream);

/* Thread-local description of the last error (empty string if none). */
const char* hum_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HUM_H_ */
