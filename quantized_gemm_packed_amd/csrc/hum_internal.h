// Internal declarations shared by the library's translation units.
//
// Packed weight layout (what hum_prepare_weight produces), per expert e:
//
//   codes : [NT][KB][64 lanes][B bytes]   NT = ceil(N/16), KB = K/128
//           B = 16 for 4-bit formats, 32 for E4M3, 24 for FP6 (the
//           canonical 6-bit stream of the lane's 32 codes, unchanged: the
//           hardware's 32-wide FP6 conversion reads it in that order).  Lane l = c + 16*lg
//           (c = column within the 16-column sub-tile, lg = 0..3) holds
//             4-bit : k = 128*kb + 32*lg + (0..31)            (32 codes)
//             E4M3  : k = 128*kb + 16*lg + (0..15) then
//                     k = 128*kb + 64 + 16*lg + (0..15)     (32 codes)
//           which is the operand order of the gfx950 MFMA instructions the
//           GEMM issues (16x16x32 bf16 per 8-k step, 16x16x128 f8f6f4).
//           INT4 / UINT4 nibbles of one 8-k step sit in one dword in the
//           order k0,k2,k4,k6 at bits 0,4,8,12 and k1,k3,k5,k7 at bits
//           16,20,24,28, so that (w >> 4j) & 0x000F000F | 0x43004300 is the
//           bf16 pair (128 + u_{2j}, 128 + u_{2j+1}).  INT4 is stored
//           offset by 8 (u = v + 8).  E2M1 keeps the canonical order (even
//           k in the low nibble).
//           b-bit integers (b = 3, 2, 1; B = 4b): the same 32 codes per lane
//           in the same element order (element j of 8-k step s is k = 32*lg
//           + 8*s + j), split into bit planes.  A 2-bit plane (b = 2, 3) is
//           two dwords: step s in dword s/2, element j at bit (j & 1) * 16 +
//           2 * (4 * (s & 1) + j / 2), so that (w >> 2i) & 0x00030003 |
//           0x43004300 is a bf16 pair.  A 1-bit plane (b = 1, 3) is one dword
//           after it: element j of step s at bit (j & 1) * 16 + 4 * s + j / 2.
//           For b = 3 the 1-bit plane holds bit 2 of each code.  Signed codes
//           are stored offset by 2^(b-1).
//   meta  : INTb/UINTb : scales [NT][NG][16] (bf16 or f32), zeros
//                        [NT][NG][8 bytes] (16 nibbles, column c at nibble c)
//           E2M1/E8M0  : scales [NT][KB4][64 lanes][4 bytes], byte i of the
//                        dword of lane l is the E8M0 code of column c and
//                        32-block lg of K-block 4*kb4 + i
//           E4M3       : scales f32 [NT*16]
//   offset terms (integer formats only): -s * (offset + z) per column and
//           K-block, where offset + z is what the bf16 (128 + u) codes carry
//           beyond the code's value (signed b-bit: 128 + 2^(b-1), unsigned:
//           128 + zero point).  As
//           bf16 hi / lo pairs, [NT][KBC][64 lanes][8] hi then the same for
//           lo, KBC = ceil(KB / 32): lane l = c + 16*lg holds K-blocks
//           32*kbc + 8*lg + (0..7) of column c -- the B operand of a 16x16x32
//           bf16 MFMA whose K runs over K-blocks.  (Zero past N and KB.)
//   global scale : f32 [E] (1.0 when absent)
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/hum.h"

namespace hum {

constexpr int kNSub = 16;     // columns per sub-tile
constexpr int kKBlk = 128;    // K per packed block

struct Layout {
  int64_t nt = 0, kb = 0, ng = 0, kb4 = 0;
  int64_t codes_per_expert = 0;   // bytes
  int64_t scales_per_expert = 0;  // bytes
  int64_t zeros_per_expert = 0;   // bytes
  int64_t kbc = 0;                // INT formats: K-block chunks of 32 (offset terms)
  int64_t co_per_expert = 0;      // bytes of offset terms (hi and lo)
  int64_t codes_off = 0, scales_off = 0, zeros_off = 0, co_off = 0, gscale_off = 0, total = 0;
  int code_bytes = 16;            // per lane per (nt, kb)
  int kb_per_group = 1;           // INT formats
  int scale_f32 = 0;              // INT formats: 1 = f32 scales, 0 = bf16
};

enum Fmt : int {
  F_INT = 0, F_MXFP4_BF16 = 1, F_FP8 = 2, F_MXFP4_MXFP8 = 3, F_MXFP4_MXFP4 = 4, F_FP8_BLOCK = 5, F_FP8_BF16 = 6,
  F_INT8_BF16 = 7, F_NVFP4_BF16 = 8, F_MXINT4_BF16 = 9, F_INT3 = 10, F_INT2 = 11, F_INT1 = 12,
  F_MXFP6_BF16 = 13, F_MXBF6_BF16 = 14
};

// MXFP6 weights (E2M3 / E3M2 codes, E8M0 per 32) x bf16 activations.
constexpr bool fmt_fp6(int f) { return f == F_MXFP6_BF16 || f == F_MXBF6_BF16; }
// Formats whose weight metadata are per-lane rows of scale bytes (E8M0 per
// 32: a dword per lane covers 4 K-blocks; NVFP4's E4M3 per 16: 2).
constexpr bool fmt_mx_meta(int f) {
  return f == F_MXFP4_BF16 || f == F_MXINT4_BF16 || f == F_MXFP4_MXFP8 || f == F_NVFP4_BF16 || fmt_fp6(f);
}

// The integer family (b-bit codes with bf16 / f32 group scales, optional
// zero points, bf16 activations): one kernel path, b = 4, 3, 2, 1.
constexpr bool fmt_int(int f) { return f == F_INT || f == F_INT3 || f == F_INT2 || f == F_INT1; }
constexpr int fmt_int_bits(int f) { return f == F_INT3 ? 3 : (f == F_INT2 ? 2 : (f == F_INT1 ? 1 : 4)); }

// Bits of an integer-family weight dtype (0 for the others), and whether
// its codes are signed.
constexpr int dtype_int_bits(int dt) {
  return (dt == HUM_INT4 || dt == HUM_UINT4) ? 4
         : (dt == HUM_INT3 || dt == HUM_UINT3) ? 3
         : (dt == HUM_INT2 || dt == HUM_UINT2) ? 2
         : (dt == HUM_INT1 || dt == HUM_UINT1) ? 1 : 0;
}
constexpr bool dtype_int_signed(int dt) {
  return dt == HUM_INT4 || dt == HUM_INT3 || dt == HUM_INT2 || dt == HUM_INT1;
}

// Formats whose activations stay bf16 (bf16 MFMA on widened weights).
constexpr bool fmt_bf16_act(int f) {
  return fmt_int(f) || f == F_MXFP4_BF16 || f == F_FP8_BF16 || f == F_INT8_BF16 || f == F_NVFP4_BF16 ||
         f == F_MXINT4_BF16 || fmt_fp6(f);
}
// 8-bit weight codes laid out for the bf16 MFMA: a lane's 32 codes of a
// K-block contiguous (k = 32 * (lane / 16) + j), per-channel f32 scales.
constexpr bool fmt_w8_bf16(int f) { return f == F_FP8_BF16 || f == F_INT8_BF16; }

// Validates the description; on failure sets the thread-local error and
// returns a non-OK status.
hum_status check_desc(const hum_weight_desc* d);
hum_status compute_layout(const hum_weight_desc* d, Layout* L);
int fmt_of(const hum_weight_desc* d);

hum_status set_error(hum_status s, const char* fmt, ...);
void clear_error();

// ---- launchers (return HUM_ERR_HIP on a launch failure) -----------------
hum_status launch_repack(const hum_weight_desc* d, const Layout& L, const void* codes,
                         const void* scales, const void* zeros, const float* gscale,
                         void* packed, void* stream);
hum_status launch_dequant(const hum_weight_desc* d, const Layout& L, const void* packed,
                          float* out, void* stream);
// sorted / sentinel (optional): rows r with sorted[r] >= sentinel (padding
// slots of grouped rows) are skipped.
hum_status launch_quant_fp8_token(int64_t m, int64_t k, const void* x, int64_t ldx,
                                  void* q, float* s, void* stream, const int32_t* sorted = nullptr,
                                  int32_t sentinel = 0);
// counts / max_m (optional): quantize only the live rows of a grouped_masked
// buffer (row r is live when r % max_m < counts[r / max_m]).
hum_status launch_quant_mxfp8(int64_t m, int64_t k, const void* x, int64_t ldx, void* q,
                              uint8_t* s, void* stream, const int32_t* counts = nullptr, int64_t max_m = 0);
hum_status launch_quant_mxfp4(int64_t m, int64_t k, const void* x, int64_t ldx, void* q,
                              uint8_t* s, void* stream, const int32_t* counts = nullptr, int64_t max_m = 0);
// The MXFP4 rule with each code written as the E4M3 byte of its value (k
// bytes per row; scales as launch_quant_mxfp4): input of the E4M3 x E2M1
// decode kernel that serves W4A4 layers at decode sizes.
hum_status launch_quant_mxfp4_wide(int64_t m, int64_t k, const void* x, int64_t ldx, void* q, uint8_t* s,
                                   void* stream);
hum_status launch_quant_fp8_group(int64_t m, int64_t k, const void* x, int64_t ldx, void* q, float* s,
                                  void* stream, const int32_t* sorted = nullptr, int32_t sentinel = 0);
hum_status launch_zero(void* p, size_t bytes, void* stream);
// tmp / tmp_bytes (optional, align_workspace_bytes(t, topk, e) of scratch):
// large routing tables are sorted by many workgroups (else one).
hum_status launch_align(const int32_t* ids, int64_t t, int32_t topk, int32_t e,
                        int32_t block_m, int32_t* sorted, int32_t* offsets, int32_t* counts,
                        int32_t* block_expert, int64_t nblocks, void* stream, void* tmp = nullptr,
                        int64_t tmp_bytes = 0);
int64_t align_workspace_bytes(int64_t t, int32_t topk, int32_t e);
// block_expert[b] = the expert whose padded segment (align's offsets[E+1])
// holds rows b*block_m.., or -1 past the last segment.
hum_status launch_block_expert(const int32_t* offsets, int32_t e, int32_t block_m, int64_t nblocks,
                               int32_t* block_expert, void* stream);
// grouped_masked layout: sorted[e * max_m + i] = that position when
// i < clamp(counts[e], 0, max_m), else the sentinel E * max_m; block b of
// block_m rows belongs to expert b * block_m / max_m, or -1 when all its
// rows are padding.
hum_status launch_masked_align(const int32_t* counts, int32_t e, int64_t max_m, int32_t block_m,
                               int32_t* sorted, int32_t* block_expert, void* stream);
// ids (optional): slots whose expert id lies outside [0, num_experts) are
// skipped (they were never computed).
hum_status launch_moe_reduce(const void* y, const float* w, int64_t t, int32_t topk,
                             int64_t h, void* out, void* stream, const int32_t* ids = nullptr,
                             int32_t num_experts = 0);

// GEMM epilogues / A-row modes
enum Epi : int { EPI_BF16 = 0, EPI_SWIGLU_BF16 = 1, EPI_SWIGLU_MXFP8 = 2, EPI_SCATTER = 3, EPI_SWIGLU_MXFP4 = 4 };
// A-row modes: dense rows; grouped rows gathered through sorted (row r
// reads a[sorted[r] / topk]); grouped rows read in sorted order (row r reads
// a[r], padding slots skipped).  The scatter epilogue implies grouped rows.
enum AMode : int { A_DIRECT = 0, A_GATHER = 1, A_SORTED = 2 };

struct GemmParams {
  // weights
  const uint8_t* codes;
  const uint8_t* wscale;
  const uint8_t* wzero;
  const float* gscale;
  int64_t codes_per_expert, scales_per_expert, zeros_per_expert;
  int nt_count, kb_count, ng, kb_per_group, kb4;
  float inv_kbg;      // 1 / kb_per_group (group of K-block kb: floor((kb + 0.5) * inv_kbg))
  int scale_f32, int_offset, has_zero;
  int64_t n;          // valid output columns (I for the SwiGLU epilogues)
  int swiglu_nt_off;  // up sub-tile offset (I / 16) for SwiGLU
  // activations
  const void* a;
  int64_t lda;        // elements (bytes for fp8)
  const void* a_scale;
  int64_t a_scale_ld; // MXFP8: scale bytes per row
  // Dense decode kernel with per-token FP8 activations: a holds the bf16 rows
  // (lda elements apart) and the kernel quantizes them itself (no a_scale)
  int a_fp8_fuse;
  // INT tile kernel: activation sums per (row, K-block) as bf16 hi / lo
  // pairs, [ceil(m/16)][kbc][64 lanes][8] hi then lo (lane l = r + 16*lg
  // holds K-blocks 32*kbc + 8*lg + (0..7) of row r: the A operand of a
  // 16x16x32 bf16 MFMA whose K runs over K-blocks), and the weight's offset
  // terms in the matching B-operand layout
  const uint8_t* a_rowsum;
  const uint8_t* wco;
  int64_t co_per_expert;
  int kbc;
  int64_t a_bytes;        // bytes of the activation buffer (< 2 GiB for buffer loads)
  int64_t a_scale_bytes;  // bytes of the MXFP8 activation scale buffer
  int64_t m;          // rows (dense) / padded sorted length (MoE)
  // MoE
  const int32_t* sorted;
  const int32_t* block_expert;
  // Grouped rows whose live blocks are a prefix of the block array: the
  // padded live row count (align's offsets[E]), read by the tile kernel to
  // spread the live tiles over all XCDs.  Null: any launched tile may be
  // live (dense layers, the masked layout).
  const int32_t* live_rows;
  int topk;
  int sentinel;
  int a_gather;       // rows gathered through sorted (set from the kernel key by launch_gemm)
  // Decode-size routing inside the gathered decode kernel (no align launch):
  // route_n <= 64 flat slots of route_ids over route_e experts; each
  // workgroup finds its 16-row block's expert and rows itself, in align's
  // order, and the workgroups of the first N-tile write the blocks' sorted
  // rows (sentinel padding), block -> expert entries and the padded live
  // row count for the GEMM after it.  Null route_ids: the align's arrays.
  const int32_t* route_ids;
  int route_n, route_e;
  int32_t* route_sorted;
  int32_t* route_bexp;
  int32_t* route_live;
  // outputs
  void* out;
  int64_t ldo;        // elements
  void* out_scale;    // MXFP8 epilogue scales, [rows][ldo/32]
  float* swiglu_f32;  // SwiGLU epilogues (optional): the fp32 values stored / requantized, [rows][n]
  const uint16_t* bias;
  float* partials;    // split-K partials, [split][m][columns] fp32
  int split_k;
  int kb_per_split;
  // Stream-K (tile kernel, dense): sk_groups workgroups share the
  // sk_tiles * kb_count K-block iterations, sk_len each; per-tile counters
  // (zero between calls) and per-workgroup partial slots
  int sk_groups, sk_tiles, sk_m_tiles;
  int64_t sk_len;
  uint32_t* sk_count;
  float* sk_part;
  int64_t sk_part_bytes;
  int n_tiles;
  int group_m;        // tile kernel: M-tiles walked together (M fastest) per N sweep
  int stream_rows;    // stream kernel: most valid rows of one 16-row tile
  // stream kernel LDS plan (bytes): weight metadata of sub-tile ns at
  // lds_meta_off + ns * lds_meta_stride, INT zero points lds_zero_off
  // further
  int lds_meta_off, lds_meta_stride, lds_zero_off;
};

enum Kind : int { KIND_TILE = 0, KIND_STREAM = 1, KIND_TILE32 = 2 };

// The decode (stream) kernel stages the activation rows of its K range in
// LDS (rows x K-blocks x 256 B for bf16, 128 B (+4 B of MX scales) for
// FP8).  Dense launches keep it within kStreamLdsDense so that several
// workgroups share a CU; a MoE launch may take up to kStreamLdsMax.
constexpr int64_t kStreamLdsDense = 128 * 1024;
constexpr int64_t kStreamLdsMax = 159 * 1024;
constexpr int64_t stream_lds_per_kb(int fmt, int rows) {
  return (int64_t)rows * (fmt_bf16_act(fmt) ? 256 : (fmt == F_MXFP4_MXFP8 ? 132 : 128));
}
// Exact LDS footprint of the stream kernel's staging for at most `rows`
// rows and `kb` K-blocks: 16-byte activation slots and 4-byte MX scale
// slots, each rounded up to whole 64-lane LDS-DMA instructions (every lane
// of an instruction writes its slot).
constexpr int64_t stream_lds_footprint(int fmt, int rows, int64_t kb) {
  const int64_t cpr = fmt_bf16_act(fmt) ? 16 : 8;
  const int64_t a = ((rows * cpr * kb + 63) / 64) * 64 * 16;
  const int64_t sc = (fmt == F_MXFP4_MXFP8) ? ((rows * kb + 63) / 64) * 64 * 4 : 0;
  return a + sc;
}

// Full LDS plan of a stream launch: the activation staging, then per
// sub-tile the weight metadata of the K range (INT: scales then zero points
// of the groups it touches; MX: the E8M0 rows of its 4-K-block steps), each
// rounded up to whole 64-lane LDS-DMA instructions.
struct StreamLdsPlan {
  int64_t meta_off, meta_stride, zero_off, total;
};
constexpr StreamLdsPlan stream_lds_plan(int fmt, int rows, int64_t kb, int wn, int64_t kb_per_group, int scale_f32,
                                        int64_t ng, int64_t kb4) {
  StreamLdsPlan L{stream_lds_footprint(fmt, rows, kb), 0, 0, 0};
  if (fmt == F_FP8_BLOCK) {
    // the group scales of the 16 tile rows per K-block, then the block
    // scales of the sub-tiles per K-block (the kernel quantizes the rows)
    L.total = L.meta_off + kb * 64 + ((kb * wn * 4 + 15) / 16) * 16;
    return L;
  }
  if (fmt_int(fmt)) {
    int64_t groups = (kb + kb_per_group - 1) / kb_per_group + 1;  // groups a range of kb blocks touches
    if (groups > ng) groups = ng;
    const int64_t sc = ((groups * 16 * (scale_f32 ? 4 : 2) + 1023) / 1024) * 1024;
    const int64_t zr = ((groups * 8 + 255) / 256) * 256;
    L.zero_off = sc;
    L.meta_stride = sc + zr;
  } else if (fmt_mx_meta(fmt)) {
    // scale rows a range of kb blocks touches (a row: 4 K-blocks, NVFP4 2)
    int64_t r = (fmt == F_NVFP4_BF16 ? kb / 2 : kb / 4) + 2;
    if (r > kb4) r = kb4;
    L.meta_stride = ((r * 256 + 1023) / 1024) * 1024;
  }
  L.total = L.meta_off + wn * L.meta_stride;
  return L;
}

// A self-staged (dense) stream workgroup: each of the kw compute waves
// copies its own K-blocks' activations (at most 8 16-byte chunks per lane)
// and weight metadata (INT: at most 1 KB of scales and 256 B of zero
// points; MX: at most 2 KB of E8M0 rows) with one pass of loads.
constexpr bool stream_self_stage_fits(int fmt, int rows, int64_t kb, int kw, int64_t kb_per_group, int scale_f32) {
  const int64_t per = (kb + kw - 1) / kw;
  const int64_t cpr = fmt_bf16_act(fmt) ? 16 : 8;
  if (rows * per * cpr > 512) return false;
  if (fmt_int(fmt)) {
    const int64_t groups = (per + kb_per_group - 1) / kb_per_group + 1;
    return groups * 16 * (scale_f32 ? 4 : 2) <= 1024 && groups * 8 <= 256;
  }
  if (fmt_mx_meta(fmt) && fmt != F_NVFP4_BF16) return (per / 4 + 2) * 256 <= 2048;
  if (fmt == F_NVFP4_BF16) return (per / 2 + 2) * 256 <= 2048;
  return true;
}

// The dense FP8 decode kernel quantizes per-token activations itself when
// each wave's K range holds at most 4 16-byte code chunks per lane.
// (Block-scaled FP8 activations are always quantized in the decode kernel,
// per row and K-block, under the same limit.)
constexpr bool stream_fp8_fuse_fits(int rows, int64_t kb, int kw) {
  return rows * ((kb + kw - 1) / kw) * 8 <= 256;
}

struct KernelKey {
  int fmt, kind, wm, wn, waves_n, waves_k, amode, epi;
  int stages;  // tile kernel: LDS pipeline stages (2 or 3); 0 for the stream kernel
  int sk = 0;  // 1: the Stream-K variant of a dense tile kernel
};

// Launches the GEMM kernel instance matching `key` (HUM_ERR_UNSUPPORTED if
// no such instance is compiled), followed by the split-K reduce kernel when
// p.split_k > 1.  Grid = m_tiles * n_tiles * split_k.
hum_status launch_gemm(const KernelKey& key, const GemmParams& p, int64_t m_tiles, int block_m,
                       void* stream);
bool gemm_instance_exists(const KernelKey& key);
// A split-K reduce kernel is compiled for this format and epilogue.
bool reduce_instance_exists(int fmt, int epi);
hum_status launch_rowsum(const void* a, int64_t lda, int64_t m, int kb_count, int kbc, uint8_t* out,
                         void* stream);

}  // namespace hum
