// C ABI entry points: description checks, packed layout, the tile / split-K
// selector, workspace carving and dispatch.  Host code only.
//
// The selector follows the idea of "Device-parameter tuning" in "Announcing
// Humming: Fast, Flexible Kernels for Quantized Inference": the shape, the
// format and the device's resources (here: 256 CUs, 160 KB LDS, wave64)
// choose a tile and split per M range, at run time, with no compilation.
#include <algorithm>
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "hum_internal.h"

namespace hum {

static thread_local char g_err[512];

hum_status set_error(hum_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = 0; }

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static inline int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

hum_status check_desc(const hum_weight_desc* d) {
  if (!d) return set_error(HUM_ERR_INVALID_ARG, "desc is NULL");
  if (d->num_experts < 1) return set_error(HUM_ERR_INVALID_ARG, "num_experts must be >= 1");
  if (d->n < 1) return set_error(HUM_ERR_INVALID_ARG, "n must be >= 1");
  if (d->k < 128 || d->k % 128) return set_error(HUM_ERR_UNSUPPORTED, "k must be a positive multiple of 128 (got %lld)", (long long)d->k);
  // k < 2^21: a sub-tile's weight stripe stays far below the 2 GiB reach of
  // a buffer resource, and K-block / group indices stay exact in fp32
  if (d->n > (int64_t)1 << 30 || d->k > (int64_t)1 << 21) return set_error(HUM_ERR_UNSUPPORTED, "n/k too large");
  if (d->has_zero_point != 0 && d->has_zero_point != 1) return set_error(HUM_ERR_INVALID_ARG, "has_zero_point must be 0/1");
  if (d->has_global_scale != 0 && d->has_global_scale != 1) return set_error(HUM_ERR_INVALID_ARG, "has_global_scale must be 0/1");
  if (d->scale_gran < HUM_SCALE_TENSOR || d->scale_gran > HUM_SCALE_BLOCK) return set_error(HUM_ERR_INVALID_ARG, "bad scale_gran");
  if (d->scale_gran == HUM_SCALE_BLOCK && (d->weight_dtype != HUM_E4M3 || d->group_size != 128))
    return set_error(HUM_ERR_UNSUPPORTED, "2-D block scales take E4M3 weights and 128 x 128 blocks");
  if ((d->act_fmt == HUM_ACT_FP8_GROUP) != (d->scale_gran == HUM_SCALE_BLOCK))
    return set_error(HUM_ERR_UNSUPPORTED, "block-scaled weights run with per-group FP8 activations (and only they)");
  if (d->scale_gran == HUM_SCALE_GROUP || d->scale_gran == HUM_SCALE_BLOCK) {
    if (d->group_size <= 0 || d->k % d->group_size) return set_error(HUM_ERR_INVALID_ARG, "group_size must divide k");
  }
  switch (d->weight_dtype) {
    case HUM_INT4:
    case HUM_UINT4:
    case HUM_INT3:
    case HUM_UINT3:
    case HUM_INT2:
    case HUM_UINT2:
    case HUM_INT1:
    case HUM_UINT1:
      if (d->scale_dtype == HUM_E8M0) {
        // MXINT4: signed INT4 codes with an E8M0 scale per 32 along K
        if (d->weight_dtype != HUM_INT4 || d->scale_gran != HUM_SCALE_GROUP || d->group_size != 32)
          return set_error(HUM_ERR_UNSUPPORTED, "integer weights with E8M0 scales are INT4 with one scale per 32 (MXINT4)");
        if (d->has_zero_point) return set_error(HUM_ERR_UNSUPPORTED, "MXINT4 takes no zero point");
        if (d->act_fmt != HUM_ACT_BF16) return set_error(HUM_ERR_UNSUPPORTED, "MXINT4 weights run with bf16 activations");
        return HUM_OK;
      }
      if (d->act_fmt != HUM_ACT_BF16) return set_error(HUM_ERR_UNSUPPORTED, "integer weights run with bf16 activations");
      if (d->scale_dtype != HUM_BF16 && d->scale_dtype != HUM_F32) return set_error(HUM_ERR_UNSUPPORTED, "integer weights take bf16 or f32 scales");
      if (d->scale_gran == HUM_SCALE_GROUP && d->group_size % 128) return set_error(HUM_ERR_UNSUPPORTED, "integer group_size must be a multiple of 128");
      if (d->has_zero_point && dtype_int_signed(d->weight_dtype))
        return set_error(HUM_ERR_UNSUPPORTED, "zero points need unsigned integer codes");
      return HUM_OK;
    case HUM_E2M1:
      if (d->scale_dtype == HUM_E4M3) {
        // NVFP4: an E4M3 scale per 16 along K (+ the f32 tensor scale)
        if (d->scale_gran != HUM_SCALE_GROUP || d->group_size != 16)
          return set_error(HUM_ERR_UNSUPPORTED, "E2M1 weights with E4M3 scales take one scale per 16 along K (NVFP4)");
        if (d->has_zero_point) return set_error(HUM_ERR_UNSUPPORTED, "E2M1 takes no zero point");
        if (d->act_fmt != HUM_ACT_BF16) return set_error(HUM_ERR_UNSUPPORTED, "NVFP4 weights run with bf16 activations");
        return HUM_OK;
      }
      if (d->scale_gran != HUM_SCALE_GROUP || d->group_size != 32 || d->scale_dtype != HUM_E8M0)
        return set_error(HUM_ERR_UNSUPPORTED, "E2M1 weights need E8M0 scales per 32 along K (MXFP4)");
      if (d->has_zero_point) return set_error(HUM_ERR_UNSUPPORTED, "E2M1 takes no zero point");
      if (d->act_fmt != HUM_ACT_BF16 && d->act_fmt != HUM_ACT_MXFP8 && d->act_fmt != HUM_ACT_MXFP4)
        return set_error(HUM_ERR_UNSUPPORTED, "MXFP4 runs with bf16, MXFP8 or MXFP4 activations");
      return HUM_OK;
    case HUM_E2M3:
    case HUM_E3M2:
      if (d->scale_gran != HUM_SCALE_GROUP || d->group_size != 32 || d->scale_dtype != HUM_E8M0)
        return set_error(HUM_ERR_UNSUPPORTED, "FP6 weights need E8M0 scales per 32 along K (MXFP6)");
      if (d->has_zero_point) return set_error(HUM_ERR_UNSUPPORTED, "FP6 takes no zero point");
      if (d->act_fmt != HUM_ACT_BF16) return set_error(HUM_ERR_UNSUPPORTED, "MXFP6 weights run with bf16 activations");
      return HUM_OK;
    case HUM_INT8:
      if (d->scale_gran != HUM_SCALE_CHANNEL && d->scale_gran != HUM_SCALE_TENSOR)
        return set_error(HUM_ERR_UNSUPPORTED, "INT8 weights take per-channel or per-tensor scales");
      if (d->scale_dtype != HUM_F32) return set_error(HUM_ERR_UNSUPPORTED, "INT8 weights take f32 scales");
      if (d->has_zero_point) return set_error(HUM_ERR_UNSUPPORTED, "INT8 takes no zero point");
      if (d->act_fmt != HUM_ACT_BF16) return set_error(HUM_ERR_UNSUPPORTED, "INT8 weights run with bf16 activations");
      return HUM_OK;
    case HUM_E4M3:
      if (d->scale_gran == HUM_SCALE_GROUP) return set_error(HUM_ERR_UNSUPPORTED, "E4M3 weights take per-channel or per-tensor scales");
      if (d->scale_dtype != HUM_F32) return set_error(HUM_ERR_UNSUPPORTED, "E4M3 weights take f32 scales");
      if (d->has_zero_point) return set_error(HUM_ERR_UNSUPPORTED, "E4M3 takes no zero point");
      if (d->act_fmt != HUM_ACT_FP8_TOKEN && d->act_fmt != HUM_ACT_FP8_GROUP && d->act_fmt != HUM_ACT_BF16)
        return set_error(HUM_ERR_UNSUPPORTED, "E4M3 weights run with per-token or per-group FP8, or bf16, activations");
      return HUM_OK;
    default:
      return set_error(HUM_ERR_UNSUPPORTED, "unsupported weight dtype %d", d->weight_dtype);
  }
}

int fmt_of(const hum_weight_desc* d) {
  if (d->weight_dtype == HUM_INT4 && d->scale_dtype == HUM_E8M0) return F_MXINT4_BF16;
  switch (dtype_int_bits(d->weight_dtype)) {
    case 4: return F_INT;
    case 3: return F_INT3;
    case 2: return F_INT2;
    case 1: return F_INT1;
    default: break;
  }
  if (d->weight_dtype == HUM_INT8) return F_INT8_BF16;
  if (d->weight_dtype == HUM_E2M3) return F_MXFP6_BF16;
  if (d->weight_dtype == HUM_E3M2) return F_MXBF6_BF16;
  if (d->weight_dtype == HUM_E4M3)
    return d->scale_gran == HUM_SCALE_BLOCK ? F_FP8_BLOCK : (d->act_fmt == HUM_ACT_BF16 ? F_FP8_BF16 : F_FP8);
  if (d->scale_dtype == HUM_E4M3) return F_NVFP4_BF16;
  if (d->act_fmt == HUM_ACT_MXFP8) return F_MXFP4_MXFP8;
  return d->act_fmt == HUM_ACT_MXFP4 ? F_MXFP4_MXFP4 : F_MXFP4_BF16;
}

hum_status compute_layout(const hum_weight_desc* d, Layout* L) {
  hum_status st = check_desc(d);
  if (st != HUM_OK) return st;
  *L = Layout();
  L->nt = cdiv(d->n, kNSub);
  L->kb = d->k / kKBlk;
  L->kb4 = cdiv(L->kb, 4);
  const int f = fmt_of(d);
  L->code_bytes = (f == F_FP8 || f == F_FP8_BLOCK || fmt_w8_bf16(f)) ? 32
                  : (fmt_int(f) ? 4 * fmt_int_bits(f) : (fmt_fp6(f) ? 24 : 16));
  L->codes_per_expert = L->nt * L->kb * 64 * L->code_bytes;
  if (fmt_int(f)) {
    const bool grp = d->scale_gran == HUM_SCALE_GROUP && d->group_size < d->k;
    L->ng = grp ? d->k / d->group_size : 1;
    L->kb_per_group = grp ? d->group_size / kKBlk : (int)L->kb;
    L->scale_f32 = d->scale_dtype == HUM_F32;
    L->scales_per_expert = align256(L->nt * L->ng * 16 * (L->scale_f32 ? 4 : 2));
    L->zeros_per_expert = d->has_zero_point ? align256(L->nt * L->ng * 8) : 0;
    L->kbc = cdiv(L->kb, 32);
    L->co_per_expert = L->nt * L->kbc * 1024 * 2;
  } else if (f == F_FP8 || fmt_w8_bf16(f)) {
    L->ng = 1;
    L->scales_per_expert = align256(L->nt * 16 * 4);
  } else if (f == F_FP8_BLOCK) {
    // one f32 per 16-column sub-tile and K-block (a sub-tile lies in one
    // 128-row block)
    L->ng = L->kb;
    L->scales_per_expert = align256(L->nt * L->kb * 4);
  } else if (f == F_NVFP4_BF16) {
    // a dword per lane and pair of K-blocks: the lane's two E4M3 group
    // scales (16 along K each) of either K-block
    L->ng = L->kb * 8;
    L->kb4 = cdiv(L->kb, 2);
    L->scales_per_expert = L->nt * L->kb4 * 64 * 4;
  } else {
    L->ng = L->kb * 4;
    L->scales_per_expert = L->nt * L->kb4 * 64 * 4;
  }
  const int64_t E = d->num_experts;
  L->codes_off = 0;
  L->scales_off = align256(E * L->codes_per_expert);
  L->zeros_off = align256(L->scales_off + E * L->scales_per_expert);
  L->co_off = align256(L->zeros_off + E * L->zeros_per_expert);
  L->gscale_off = align256(L->co_off + E * L->co_per_expert);
  L->total = align256(L->gscale_off + E * 4);
  return HUM_OK;
}

// ---------------------------------------------------------------------------
// Selector.

static const int kCUs = 256;

static int key_stages(const hum_tile_config& c) {
  return c.kind != HUM_KERNEL_STREAM ? (c.stages == 0 ? 2 : c.stages) : 0;
}

// W4A4 on the decode kernel runs as E4M3 x E2M1: its MXFP4 activations are
// quantized as the E4M3 bytes of the same values.
static bool w4a4_on_stream(const hum_weight_desc* d, const hum_tile_config& c) {
  return fmt_of(d) == F_MXFP4_MXFP4 && c.kind == HUM_KERNEL_STREAM;
}

static KernelKey dense_key(const hum_weight_desc* d, const hum_tile_config& c) {
  return KernelKey{w4a4_on_stream(d, c) ? (int)F_MXFP4_MXFP8 : fmt_of(d), c.kind, c.wave_m, c.wave_n, c.waves_n,
                   c.waves_k, A_DIRECT, EPI_BF16, key_stages(c), c.stream_k > 0 ? 1 : 0};
}

// Stream-K tile counters: the workspace header, one u32 per tile.
constexpr int64_t kWsHeader = HUM_WS_HEADER_BYTES;
constexpr int64_t kSkMaxTiles = kWsHeader / 4;

static bool cfg_sane(const hum_tile_config& c) {
  if (c.split_k < 1 || c.split_k > 64 || c.wave_m < 1 || c.wave_n < 1) return false;
  if (c.stream_k < 0 || c.stream_k > 65536) return false;
  if (c.stream_k > 0 && (c.kind == HUM_KERNEL_STREAM || c.split_k != 1)) return false;
  if (c.kind == HUM_KERNEL_STREAM) return c.wave_m == 1 && c.waves_n == 1 && c.waves_k >= 1 && c.waves_k <= 15;
  if (c.kind == HUM_KERNEL_TILE) return c.waves_n == 4 && c.waves_k == 1 && (c.stages == 0 || c.stages == 2 || c.stages == 3);
  if (c.kind == HUM_KERNEL_TILE32)
    return c.waves_n == 4 && c.waves_k == 1 && (c.stages == 0 || c.stages == 2 || c.stages == 3) && c.wave_m % 2 == 0 &&
           c.wave_n % 2 == 0;
  return false;
}

static int64_t tile_rows(const hum_tile_config& c) { return 16 * (int64_t)c.wave_m; }

// Columns (16-wide sub-tiles) one workgroup covers.
static int64_t tile_subtiles(const hum_tile_config& c) {
  return (int64_t)c.wave_n * (c.kind != HUM_KERNEL_STREAM ? 4 : 1);
}

// Grid split so that the launch reaches `target` waves, each split keeping
// at least min_kb K-blocks per wave.
static int pick_split(int64_t wgs, int waves_per_wg, int64_t kb, int k_waves, int min_kb, int64_t target_waves) {
  int s = 1;
  while (wgs * s * waves_per_wg < target_waves && kb / ((int64_t)k_waves * s * 2) >= min_kb && s < 16) s *= 2;
  return s;
}

// K-blocks per split: whole stages (waves_k K-blocks per wave-step).
static int kb_per_split(int64_t kb, const hum_tile_config& c) {
  const int64_t unit = c.kind == HUM_KERNEL_STREAM ? c.waves_k : 1;
  return (int)(cdiv(cdiv(kb, c.split_k), unit) * unit);
}

// fused_decode: the activations are bf16 (not pre-quantized), so W4A4 and
// block-scaled FP8 may take the decode kernel, which quantizes them itself.
static hum_tile_config select_dense(const hum_weight_desc* d, int64_t m, bool fused_decode = true) {
  if (fused_decode && fmt_of(d) == F_MXFP4_MXFP4 && m <= 16) {
    // W4A4 at decode sizes: the E4M3 x E2M1 decode kernel, one sub-tile and
    // four K-waves per workgroup while the activation rows fit its LDS
    // (measured at N = 7168, K = 2048: M = 1 8.1 us, M = 16 10.6 us against
    // 11.5 and 11.9 on the 32 x 128 tile; two or four sub-tiles with eight
    // K-waves 10-20% slower)
    hum_tile_config c{};
    c.kind = HUM_KERNEL_STREAM;
    c.wave_m = 1;
    c.wave_n = 1;
    c.waves_n = 1;
    c.waves_k = 4;
    c.split_k = 1;
    c.block_m = 16;
    Layout L;
    compute_layout(d, &L);
    if (stream_lds_plan(F_MXFP4_MXFP8, (int)m, kb_per_split(L.kb, c), 1, L.kb_per_group, L.scale_f32, L.ng, L.kb4)
            .total <= kStreamLdsDense)
      return c;
  }
  hum_tile_config c{};
  const int64_t nt = cdiv(d->n, kNSub);
  const int64_t kb = d->k / kKBlk;
  if (fused_decode && fmt_of(d) == F_FP8_BLOCK && m <= 16) {
    // block-scaled FP8 at decode sizes: the decode kernel, which quantizes
    // each row's K-blocks itself, wherever the per-token FP8 layer of the
    // same shape takes it and the rows fit four code chunks per lane
    hum_weight_desc dt = *d;
    dt.scale_gran = HUM_SCALE_CHANNEL;
    dt.group_size = 0;
    dt.act_fmt = HUM_ACT_FP8_TOKEN;
    const hum_tile_config ct = select_dense(&dt, m);
    if (ct.kind == HUM_KERNEL_STREAM && stream_fp8_fuse_fits((int)m, kb_per_split(kb, ct), ct.waves_k)) return ct;
  }
  if (m <= 16 && fmt_of(d) != F_MXFP4_MXFP4 && fmt_of(d) != F_FP8_BLOCK) {
    // decode: one 16-row tile streamed by waves splitting K.  Sub-tiles per
    // wave: the fewest that keep the activation bytes each workgroup reads
    // (from L2) at or below its weight bytes.  Four K-waves when their K
    // ranges fit the self-staging limits without more split-K, else eight
    // (measured on MI355X: INT M = 1, FP8 M = 1..16 run best on four).
    c.kind = HUM_KERNEL_STREAM;
    c.wave_m = 1;
    c.waves_n = 1;
    const bool bf16_act = fmt_bf16_act(fmt_of(d));
    const int64_t a_bytes = m * (bf16_act ? 2 : 1);            // per k
    const int64_t w_bytes16 = (fmt_of(d) == F_FP8 || fmt_w8_bf16(fmt_of(d)))
                                  ? 16
                                  : (fmt_int(fmt_of(d)) ? 2 * fmt_int_bits(fmt_of(d))
                                                        : (fmt_fp6(fmt_of(d)) ? 12 : 8));  // per k of a 16-column sub-tile
    const int64_t need = cdiv(a_bytes, w_bytes16);
    // (weights of 4 bits and fewer: four sub-tiles as soon as one is not
    // enough -- measured at M = 8, N = K = 8192: 16 us against 24 with two)
    // At M <= 4 one sub-tile per wave keeps enough workgroups to go without
    // split-K for every format (3- and 2-bit weights would otherwise take two)
    c.wave_n = (need <= 1 || m <= 4) ? 1 : ((need <= 2 && w_bytes16 > 8) ? 2 : 4);
    const int64_t wgs = cdiv(nt, c.wave_n);
    Layout L;
    compute_layout(d, &L);
    auto fits = [&](const hum_tile_config& t) {
      // (MXFP8 activations are staged by a loader wave, whole split at once)
      return stream_lds_plan(fmt_of(d), (int)m, kb_per_split(kb, t), t.wave_n, L.kb_per_group, L.scale_f32, L.ng,
                             L.kb4).total <= kStreamLdsDense &&
             (fmt_of(d) == F_MXFP4_MXFP8 ||
              stream_self_stage_fits(fmt_of(d), (int)m, kb_per_split(kb, t), t.waves_k, L.kb_per_group, L.scale_f32));
    };
    c.waves_k = 8;
    c.split_k = pick_split(wgs, 8, kb, 8, 2, 16 * kCUs);
    hum_tile_config c4 = c;
    c4.waves_k = 4;
    if (gemm_instance_exists(dense_key(d, c4)) && fits(c4)) {
      c = c4;
    } else {
      while (c.split_k < 64 && !fits(c)) c.split_k *= 2;
    }
    if (m > 4 && c.split_k > 1) {
      // Where the decode kernel needs split-K (and its reduce launch), the
      // 32 x 128 tile with Stream-K over 256 workgroups is faster despite
      // its unused rows (measured at M = 16, N = K = 8192: UINT4 17.5 us
      // against 24, MXFP4 14.3 against 22; at M = 5..8: UINT4 18.0 against
      // 23.3, MXFP4 13.5 against 21.4); MXFP4 takes the 16 x 128 tile
      // (13.5 us against 14.4 for 32 x 128)
      hum_tile_config t{};
      t.kind = HUM_KERNEL_TILE;
      t.wave_m = fmt_of(d) == F_MXFP4_BF16 ? 1 : 2;
      t.wave_n = 2;
      t.waves_n = 4;
      t.waves_k = 1;
      t.split_k = 1;
      t.stages = 3;
      t.stream_k = 256;
      if (gemm_instance_exists(dense_key(d, t))) c = t;
    }
  } else {
    c.kind = HUM_KERNEL_TILE;
    c.waves_n = 4;
    c.waves_k = 1;
    // Measured on MI355X (dense N = K = 8192 and N = 7168, K = 2048): small
    // tiles with split-K while the tile count is low; 64 x 256 tiles for
    // bf16 activations from M = 512 (fewer LDS activation reads per MFMA);
    // 128 x 128 for FP8 activations.  W4A4 and block-scaled FP8 come here
    // from M = 1 where their decode-kernel paths do not apply.
    const bool bf16_act = fmt_bf16_act(fmt_of(d));
    int64_t target = 3 * kCUs;
    if (m <= 256) {
      c.wave_m = 2;
      c.wave_n = 2;
      c.stages = 3;  // small tiles: room in LDS for a deeper pipeline
      if (bf16_act) target = 8 * kCUs;
    } else if (bf16_act) {
      // (8-bit weights: 64 x 128 at every M, measured at N = 7168, K =
      // 2048: 116 us against 122 for 64 x 256 at M = 4096)
      c.wave_m = 4;
      c.wave_n = (m >= 512 && !fmt_w8_bf16(fmt_of(d))) ? 4 : 2;
    } else {
      // per-channel FP8: 64 x 128 below M = 1024, 128 x 128 from there
      // (measured at N = 7168, K = 2048: M = 512 22.4 us against 24.4, M =
      // 768 even, M = 1024 29.9 against 32.4)
      c.wave_m = (fmt_of(d) == F_FP8 && m < 1024) ? 4 : 8;
      c.wave_n = 2;
    }
    const int64_t wgs = cdiv(m, tile_rows(c)) * cdiv(nt, tile_subtiles(c));
    // 8-bit weights with bf16 activations: split K only while every split
    // keeps at least 16 K-blocks (so none at K = 2048, where one pass
    // measured 1.6-2.4x faster than split-K for M = 64..256 on MI355X)
    c.split_k = pick_split(wgs, 4, kb, 1, fmt_w8_bf16(fmt_of(d)) ? 16 : 4, target);
    if (fmt_of(d) == F_FP8_BLOCK) {
      // block-scaled FP8 above decode sizes: small tiles with three stages
      // to M = 256, then the FP8 128 x 128 tiles
      if (m <= 256) {
        c.wave_m = 2;
        c.wave_n = 2;
        c.stages = 3;
      }
      c.split_k = 1;
    }
    if ((fmt_int(fmt_of(d)) && m >= 256) || (fmt_of(d) == F_MXFP4_BF16 && m >= 512)) {
      // INT / MXFP4 weights with bf16 activations: 32 x 32 MFMA blocks (the
      // bf16 16x16x32 shape issues at about half the 32x32x16 rate).
      // Measured on MI355X at N = K = 8192: INT 64 x 128 tiles with three
      // stages at M = 256, 64 x 256 with three stages to M = 1024 and two
      // above; MXFP4 64 x 256 with three stages to M = 1024, 128 x 256 with
      // two above
      c.kind = HUM_KERNEL_TILE32;
      c.wave_m = 4;
      c.wave_n = (fmt_int(fmt_of(d)) && m < 512) ? 2 : 4;
      c.stages = m <= 1024 ? 3 : 2;
      if (fmt_of(d) == F_MXFP4_BF16 && m > 1024) c.wave_m = 8;
      c.split_k = 1;
    }
    if (fmt_of(d) == F_MXFP4_MXFP4) {
      // W4A4 (N = 7168, K = 2048): three stages throughout, 32 x 128 tiles
      // to M = 256 and 64 x 256 above, no split-K (its reduce launch costs
      // more than the parallelism gains at these weight sizes)
      c.wave_m = m <= 256 ? 2 : 4;
      c.wave_n = m <= 256 ? 2 : 4;
      c.stages = 3;
      c.split_k = 1;
    }
  }
  if (c.kind == HUM_KERNEL_TILE && m > 128) {
    // bf16-activation formats whose dequantization is heavier (NVFP4, MXINT4,
    // INT8) on 16x16 blocks: more rows per tile, measured on MI355X at N = K
    // = 8192 (INT8: N = 7168, K = 2048).  NVFP4 / MXINT4: 64 x 128 with three
    // stages at M = 256 (70.5 -> 66.4 / 78.5 -> 69.1 us), 128 x 128 to M =
    // 1024 (1024: 152 -> 134 / 177 -> 139), 128 x 256 from M = 2048 (4096:
    // 538 -> 425 / 586 -> 442); INT8 128 x 128 above M = 256 (1024: 43.5 ->
    // 39.3, 4096: 130 -> 126).  (MXFP6 measured slower on 64 x 128 at M =
    // 256 and keeps its tiles.)
    // Only where the larger tiles still number at least 3/4 of the compute
    // units (a narrow layer keeps its smaller or split tiles).
    const int f = fmt_of(d);
    const bool nv_mxi = f == F_NVFP4_BF16 || f == F_MXINT4_BF16;
    hum_tile_config b = c;
    b.split_k = 1;
    if (nv_mxi && m <= 256) {
      b.wave_m = 4;
      b.wave_n = 2;
      b.stages = 3;
    } else if (nv_mxi && m > 256) {
      b.wave_m = 8;
      b.wave_n = m >= 2048 ? 4 : 2;
      b.stages = 0;
    } else if (f == F_INT8_BF16 && m > 256) {
      b.wave_m = 8;
      b.wave_n = 2;
      b.stages = 0;
    }
    if (cdiv(m, tile_rows(b)) * cdiv(nt, tile_subtiles(b)) >= kCUs * 3 / 4 &&
        gemm_instance_exists(dense_key(d, b)))
      c = b;
  }
  if (c.kind == HUM_KERNEL_TILE && c.split_k > 1) {
    // Stream-K in place of split-K: 512 workgroups share the tiles'
    // K-blocks evenly and the last to finish a shared tile sums it, so no
    // reduce launch follows (measured on MI355X, W4A16 at N = K = 8192: M =
    // 32 / 64 / 128 in 20 / 24 / 32 us against 26 / 27 / 37 with split-K;
    // 256 workgroups at M = 32, 512 above)
    hum_tile_config sk = c;
    sk.split_k = 1;
    sk.stream_k = m <= 32 ? 256 : 512;
    const int64_t tiles = cdiv(m, tile_rows(sk)) * cdiv(nt, tile_subtiles(sk));
    if (tiles <= kSkMaxTiles && gemm_instance_exists(dense_key(d, sk))) c = sk;
  }
  c.block_m = (int32_t)tile_rows(c);
  return c;
}

// The gate_up and down GEMMs of a MoE layer may run different kernels; they
// share the expert block size (one align).
struct MoeCfg {
  hum_tile_config up, dn;
};

static hum_tile_config moe_stream_cfg() {
  hum_tile_config c{};
  c.kind = HUM_KERNEL_STREAM;
  c.wave_m = 1; c.wave_n = 4; c.waves_n = 1; c.waves_k = 8; c.split_k = 1;
  c.block_m = (int32_t)tile_rows(c);
  return c;
}

static hum_tile_config moe_tile_cfg(int wm) {
  hum_tile_config c{};
  c.kind = HUM_KERNEL_TILE;
  c.wave_m = wm; c.wave_n = 4; c.waves_n = 4; c.waves_k = 1; c.split_k = 1;
  c.block_m = (int32_t)tile_rows(c);
  return c;
}

// 16-row tiles of 128 columns with three stages: twice the workgroups of
// the 256-column tile, two K-blocks in flight.  The down GEMM of decode-size
// layers (measured at T = 1, E = 128, top-8, H = 4096, I = 1024: layer W4A16
// 23.0 -> 21.0 us, W4A8 24.5 -> 22.0, W4A4 26.2 -> 24.0; 64-column tiles no
// better), and both GEMMs wherever MXFP4 x bf16 and block-scaled FP8 layers
// take 16-row tiles (W4A16 T = 2 / 4 / 16 / 64: 45.5 -> 31.7, 54.8 -> 46.5,
// 115 -> 110, 164 -> 159 us; block FP8 T = 1: 47.5 -> 33.3 us)
static hum_tile_config moe_tile16_cfg() {
  hum_tile_config c = moe_tile_cfg(1);
  c.wave_n = 2;
  c.stages = 3;
  return c;
}

// Expert weight formats the MoE layers run (per activation format).
static bool moe_fmt_ok(int f) {
  return f == F_MXFP4_BF16 || f == F_MXFP4_MXFP8 || f == F_MXFP4_MXFP4 || f == F_MXINT4_BF16 || f == F_NVFP4_BF16 ||
         f == F_FP8 || f == F_FP8_BLOCK || f == F_FP8_BF16 || f == F_INT8_BF16;
}

// The gate_up GEMM's epilogue for a format.
static int moe_up_epi(int f) {
  return f == F_MXFP4_MXFP8 ? EPI_SWIGLU_MXFP8 : (f == F_MXFP4_MXFP4 ? EPI_SWIGLU_MXFP4 : EPI_SWIGLU_BF16);
}

// The format a MoE GEMM of format f runs on the decode kernel: W4A4 gate_up
// runs there as E4M3 x E2M1 (its MXFP4 activations handed over as the E4M3
// bytes of the same values, requantized to MXFP4 in the SwiGLU epilogue).
static int moe_stream_fmt(int f) { return f == F_MXFP4_MXFP4 ? F_MXFP4_MXFP8 : f; }

// A gathered decode-kernel configuration stages the activation rows of its
// whole K range (and the weight metadata) in LDS: it fits when that plan and
// the in-workgroup reduction stay within kStreamLdsMax.
static bool moe_stream_fits(const hum_weight_desc* w, const hum_tile_config& c, int rows) {
  if (c.kind != HUM_KERNEL_STREAM) return true;
  Layout L;
  if (compute_layout(w, &L) != HUM_OK) return false;
  const StreamLdsPlan P = stream_lds_plan(moe_stream_fmt(fmt_of(w)), rows, kb_per_split(L.kb, c), c.wave_n,
                                         L.kb_per_group, L.scale_f32, L.ng, L.kb4);
  const int64_t red = (int64_t)(c.waves_k - 1) * c.wave_n * 64 * 16;
  return P.total <= kStreamLdsMax && red <= kStreamLdsMax;
}

// Makes a decode-kernel GEMM of the layer fit its LDS plan: more split-K
// (where a reduce exists) while the K range is too long, else the 16-row
// tile kernel for both GEMMs.
static void moe_fit(const hum_weight_desc* w13, const hum_weight_desc* w2, int64_t t, int32_t topk, MoeCfg& mc) {
  const int rows = (int)(t * topk < 16 ? t * topk : 16);
  const int f = fmt_of(w13);
  const int epi_up = moe_up_epi(f);
  auto fix = [&](const hum_weight_desc* w, hum_tile_config& c, int epi) -> bool {
    while (!moe_stream_fits(w, c, rows)) {
      if (c.split_k >= 8 || !reduce_instance_exists(f, epi)) return false;
      c.split_k *= 2;
    }
    return true;
  };
  if (!fix(w13, mc.up, epi_up) || !fix(w2, mc.dn, EPI_SCATTER)) mc = MoeCfg{moe_tile_cfg(1), moe_tile_cfg(1)};
}

// Measured on MI355X (E = 128, top-8, H = 4096, I = 1024, MXFP4 weights with
// bf16 or MXFP8 activations). The tile kernels read each routed expert's
// weights once per 16 or 32 rows on MFMA and win as soon as their grid
// (routed experts times 256-column slabs of the gate/up GEMM) covers half the
// CUs; below that (one token, eight experts) the decode kernel, which also
// splits K across workgroups, is faster.  Then, for bf16 activations over
// uniform routing, 16-row tiles below 8 mean rows per expert, 32 below 128,
// 64 below 512 and 128 beyond; with FP8 activations, measured over
// Zipf-skewed routing (the hot experts hold many times the mean), 16-row
// tiles below 4, 32-row tiles to 96, 64-row tiles beyond.
static MoeCfg select_moe_shape(const hum_weight_desc* w13, int64_t t, int32_t topk);
static MoeCfg select_moe(const hum_weight_desc* w13, int64_t t, int32_t topk, const hum_weight_desc* w2 = nullptr) {
  MoeCfg mc = select_moe_shape(w13, t, topk);
  if (w2) moe_fit(w13, w2, t, topk, mc);
  return mc;
}

static MoeCfg select_moe_shape(const hum_weight_desc* w13, int64_t t, int32_t topk) {
  const double rows = (double)t * topk / w13->num_experts;
  const int f = fmt_of(w13);
  if (f == F_MXFP4_MXFP4 && t * topk <= 64) {
    // W4A4 up to 64 routed slots: gate_up on the E4M3 x E2M1 decode kernel
    // with four K-waves (as W4A8), down on the 16-row W4A4 tile
    hum_tile_config up = moe_stream_cfg();
    up.waves_k = 4;
    return {up, moe_tile16_cfg()};
  }
  if ((f == F_MXFP4_MXFP4 || (f == F_MXFP4_MXFP8 && t * topk > 64)) && rows < 4) {
    // MX-activation layers below 4 mean rows per expert (past the decode
    // path of W4A8 and W4A4): 16-row tiles with three stages, gate_up 256
    // columns wide (its MX requantization takes 32-column blocks), down 128
    // (measured with Zipf-skewed routing, E = 128, top-8, H = 4096, I =
    // 1024: W4A8 T = 16 59.2 -> 52.0 us, W4A4 61.1 -> 53.9; at 4 mean rows
    // the hot experts' many 16-row blocks lost to 32-row tiles on one
    // routing, 83.7 -> 89.1 us, and won on another, 81.2 -> 77.7)
    hum_tile_config up = moe_tile_cfg(1);
    up.stages = 3;
    return {up, moe_tile16_cfg()};
  }
  if (f == F_MXFP4_MXFP4 || f == F_FP8_BLOCK) {
    // W4A4 and block-scaled FP8: tile kernels (block-scaled FP8 has no
    // decode-kernel path);
    // measured over Zipf-skewed routing like the FP8-activation rule below,
    // block-scaled FP8 taking 64-row tiles from 24 rows per expert
    const int wm = rows < 4 ? 1 : (rows <= (f == F_FP8_BLOCK ? 24 : 96) ? 2 : 4);
    if (f == F_FP8_BLOCK && wm == 1) return {moe_tile16_cfg(), moe_tile16_cfg()};
    return {moe_tile_cfg(wm), moe_tile_cfg(wm)};
  }
  const int64_t tile_wgs = std::min<int64_t>(t * topk, w13->num_experts) * cdiv(w13->n, 256);
  // MXFP4 experts with bf16 activations at one token, or with MXFP8
  // activations up to 64 routed slots (Zipf-skewed routing): gate_up on the
  // decode kernel with four K-waves per workgroup (eight waves of one or two
  // K-blocks each spent more time in their fixed costs than in their loads),
  // down on the 16-row tile kernel.  Measured per GEMM at T = 1 (bf16):
  // gate_up 15.2 -> 12.9 us, down 17.2 -> 10.3 us.
  if ((f == F_MXFP4_BF16 && tile_wgs < 128) || (f == F_MXFP4_MXFP8 && t * topk <= 64)) {
    hum_tile_config up = moe_stream_cfg();
    up.waves_k = 4;
    return {up, moe_tile16_cfg()};
  }
  if (tile_wgs < 128) return {moe_stream_cfg(), moe_stream_cfg()};
  const bool fp8_act = f == F_MXFP4_MXFP8 || f == F_FP8;
  const int wm = fp8_act ? (rows < 4 ? 1 : (rows <= 96 ? 2 : 4))
                         : (rows < 8 ? 1 : (rows < 128 ? 2 : (rows < 512 ? 4 : 8)));
  hum_tile_config c = (f == F_MXFP4_BF16 && wm == 1) ? moe_tile16_cfg() : moe_tile_cfg(wm);
  // W4A8 32- and 64-row tiles: three stages (the down GEMM has only 8
  // K-blocks, and a second block in flight hides more of each one's load
  // latency; about 4% on the layer from T = 256 to 8192)
  if (f == F_MXFP4_MXFP8 && wm >= 2) c.stages = 3;
  return {c, c};
}

static void log_cfg(const char* what, const hum_tile_config& c, int64_t m) {
  static int on = -1;
  if (on < 0) {
    const char* e = getenv("HUM_LOG");
    on = e && e[0] == '1';
  }
  if (on)
    fprintf(stderr, "[hum] %s m=%lld kind=%d wave_m=%d wave_n=%d waves_n=%d waves_k=%d split_k=%d block_m=%d\n",
            what, (long long)m, c.kind, c.wave_m, c.wave_n, c.waves_n, c.waves_k, c.split_k, c.block_m);
}

// ---------------------------------------------------------------------------
// Dense workspace: [split-K partials][quantized activations][scales][row sums].

struct DenseWs {
  int64_t partials = 0, aq = 0, as = 0, rowsum = 0, total = 0;
};

static DenseWs dense_ws(const hum_weight_desc* d, int64_t m, const hum_tile_config& c, bool quant_a) {
  DenseWs w;
  const int64_t nt = cdiv(d->n, kNSub);
  int64_t off = kWsHeader;  // Stream-K tile counters
  w.partials = off;
  if (c.split_k > 1) off = align256(off + (int64_t)c.split_k * m * nt * 16 * 4);
  // Stream-K: two partial-tile slots per workgroup
  if (c.stream_k > 0) off = align256(off + 2 * (int64_t)c.stream_k * tile_rows(c) * tile_subtiles(c) * 16 * 4);
  w.aq = off;
  if (quant_a) {
    off = align256(off + (d->act_fmt == HUM_ACT_MXFP4 && !w4a4_on_stream(d, c) ? m * (d->k / 2) : m * d->k));
    w.as = off;
    off = align256(off + (d->act_fmt == HUM_ACT_MXFP8 || d->act_fmt == HUM_ACT_MXFP4
                              ? m * (d->k / 32)
                              : (d->act_fmt == HUM_ACT_FP8_GROUP ? m * (d->k / 128) * 4 : m * 4)));
  }
  w.rowsum = off;
  if (fmt_int(fmt_of(d)) && c.kind != HUM_KERNEL_STREAM) off = align256(off + cdiv(m, 16) * cdiv(d->k / kKBlk, 32) * 2048);
  // a call that uses no scratch at all needs no workspace
  w.total = off == kWsHeader && c.stream_k == 0 ? 0 : off;
  return w;
}

}  // namespace hum

using namespace hum;

extern "C" {

const char* hum_last_error(void) { return g_err; }

size_t hum_packed_weight_bytes(const hum_weight_desc* desc) {
  clear_error();
  Layout L;
  if (compute_layout(desc, &L) != HUM_OK) return 0;
  return (size_t)L.total;
}

hum_status hum_prepare_weight(const hum_weight_desc* desc, const void* codes, const void* scales,
                              const void* zeros, const float* global_scale, void* packed,
                              size_t packed_bytes, void* stream) {
  clear_error();
  Layout L;
  hum_status st = compute_layout(desc, &L);
  if (st != HUM_OK) return st;
  if (!codes || !scales || !packed) return set_error(HUM_ERR_INVALID_ARG, "codes, scales and packed must be non-NULL");
  if (desc->has_zero_point && !zeros) return set_error(HUM_ERR_INVALID_ARG, "zeros is NULL but has_zero_point = 1");
  if (desc->has_global_scale && !global_scale) return set_error(HUM_ERR_INVALID_ARG, "global_scale is NULL but has_global_scale = 1");
  if (packed_bytes < (size_t)L.total) return set_error(HUM_ERR_WORKSPACE, "packed buffer too small (%zu < %lld)", packed_bytes, (long long)L.total);
  return launch_repack(desc, L, codes, scales, zeros, global_scale, packed, stream);
}

hum_status hum_dequant_weight(const hum_weight_desc* desc, const void* packed, float* out, void* stream) {
  clear_error();
  Layout L;
  hum_status st = compute_layout(desc, &L);
  if (st != HUM_OK) return st;
  if (!packed || !out) return set_error(HUM_ERR_INVALID_ARG, "packed and out must be non-NULL");
  return launch_dequant(desc, L, packed, out, stream);
}

hum_status hum_quant_act(int32_t act_fmt, int64_t m, int64_t k, const void* x_bf16, int64_t ld_x, void* q,
                         void* scales, void* stream) {
  clear_error();
  if (m < 0 || k <= 0 || ld_x < k) return set_error(HUM_ERR_INVALID_ARG, "bad m/k/ld_x");
  if (m > 0 && (!x_bf16 || !q || !scales)) return set_error(HUM_ERR_INVALID_ARG, "NULL pointer");
  if (k % 8 || ld_x % 8) return set_error(HUM_ERR_UNSUPPORTED, "k and ld_x must be multiples of 8");
  if (act_fmt == HUM_ACT_FP8_TOKEN) return launch_quant_fp8_token(m, k, x_bf16, ld_x, q, static_cast<float*>(scales), stream);
  if (act_fmt == HUM_ACT_MXFP8) {
    if (k % 32) return set_error(HUM_ERR_UNSUPPORTED, "MXFP8 needs k % 32 == 0");
    return launch_quant_mxfp8(m, k, x_bf16, ld_x, q, static_cast<uint8_t*>(scales), stream);
  }
  if (act_fmt == HUM_ACT_MXFP4) {
    if (k % 32) return set_error(HUM_ERR_UNSUPPORTED, "MXFP4 needs k % 32 == 0");
    return launch_quant_mxfp4(m, k, x_bf16, ld_x, q, static_cast<uint8_t*>(scales), stream);
  }
  if (act_fmt == HUM_ACT_FP8_GROUP) {
    if (k % 128) return set_error(HUM_ERR_UNSUPPORTED, "FP8_GROUP needs k % 128 == 0");
    return launch_quant_fp8_group(m, k, x_bf16, ld_x, q, static_cast<float*>(scales), stream);
  }
  return set_error(HUM_ERR_INVALID_ARG, "act_fmt must be FP8_TOKEN, MXFP8, MXFP4 or FP8_GROUP");
}

hum_status hum_select_config(const hum_weight_desc* desc, int64_t m, hum_tile_config* cfg_out) {
  clear_error();
  hum_status st = check_desc(desc);
  if (st != HUM_OK) return st;
  if (!cfg_out || m < 0) return set_error(HUM_ERR_INVALID_ARG, "bad arguments");
  *cfg_out = select_dense(desc, m < 1 ? 1 : m);
  return HUM_OK;
}

// Batch invariance: the tile kernel sums every output row in one fixed
// order (K-blocks in sequence, each through the same MFMA chain, scales
// applied per row / column), whatever its tile shape and the other rows of
// the call; split-K and the decode kernel's in-workgroup K split change that
// order.  So the invariant choice keeps the selector's tile shape for m and
// drops split-K, and replaces the decode kernel with the small-M tile.
static hum_tile_config select_dense_invariant(const hum_weight_desc* d, int64_t m) {
  hum_tile_config c = select_dense(d, m);
  if (c.kind == HUM_KERNEL_STREAM) c = select_dense(d, 17);
  // 32x32 blocks sum each dot product in another order than 16x16 ones:
  // one block shape for every m
  if (c.kind == HUM_KERNEL_TILE32) c.kind = HUM_KERNEL_TILE;
  c.split_k = 1;
  c.stream_k = 0;  // (its segments follow the tile count, hence m)
  c.block_m = (int32_t)tile_rows(c);
  return c;
}

hum_status hum_select_config_ex(const hum_weight_desc* desc, int64_t m, uint32_t flags, hum_tile_config* cfg_out) {
  clear_error();
  hum_status st = check_desc(desc);
  if (st != HUM_OK) return st;
  if (!cfg_out || m < 0) return set_error(HUM_ERR_INVALID_ARG, "bad arguments");
  if (flags & ~(uint32_t)HUM_SELECT_BATCH_INVARIANT) return set_error(HUM_ERR_INVALID_ARG, "unknown selection flags 0x%x", flags);
  *cfg_out = (flags & HUM_SELECT_BATCH_INVARIANT) ? select_dense_invariant(desc, m < 1 ? 1 : m)
                                                   : select_dense(desc, m < 1 ? 1 : m);
  return HUM_OK;
}

size_t hum_linear_workspace_bytes_ex(const hum_weight_desc* desc, int64_t m, const hum_tile_config* cfg) {
  clear_error();
  if (check_desc(desc) != HUM_OK || m < 0) return 0;
  const hum_tile_config c = cfg ? *cfg : select_dense(desc, m < 1 ? 1 : m);
  return (size_t)dense_ws(desc, m < 1 ? 1 : m, c, desc->act_fmt != HUM_ACT_BF16).total;
}

size_t hum_linear_workspace_bytes(const hum_weight_desc* desc, int64_t m) {
  return hum_linear_workspace_bytes_ex(desc, m, nullptr);
}

hum_status hum_prepare_workspace(void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  if (ws_bytes == 0) return HUM_OK;
  if (!workspace) return set_error(HUM_ERR_INVALID_ARG, "workspace is NULL");
  return launch_zero(workspace, ws_bytes, stream);
}

static void fill_weight_params(GemmParams& p, const hum_weight_desc* d, const Layout& L, const void* packed) {
  const uint8_t* pk = static_cast<const uint8_t*>(packed);
  p.codes = pk + L.codes_off;
  p.wscale = pk + L.scales_off;
  p.wzero = d->has_zero_point ? pk + L.zeros_off : nullptr;
  p.gscale = reinterpret_cast<const float*>(pk + L.gscale_off);
  p.codes_per_expert = L.codes_per_expert;
  p.scales_per_expert = L.scales_per_expert;
  p.zeros_per_expert = L.zeros_per_expert;
  p.nt_count = (int)L.nt;
  p.kb_count = (int)L.kb;
  p.ng = (int)L.ng;
  p.kb_per_group = L.kb_per_group;
  p.inv_kbg = 1.0f / (float)L.kb_per_group;
  p.kb4 = (int)L.kb4;
  p.scale_f32 = L.scale_f32;
  p.int_offset = dtype_int_signed(d->weight_dtype) ? 128 + (1 << (dtype_int_bits(d->weight_dtype) - 1)) : 128;
  p.has_zero = d->has_zero_point;
  p.n = d->n;
  p.swiglu_nt_off = 0;
  p.a_rowsum = nullptr;
  p.wco = pk + L.co_off;
  p.co_per_expert = L.co_per_expert;
  p.kbc = (int)L.kbc;
}


hum_status hum_linear_ex(const hum_weight_desc* desc, const void* packed, int64_t m, const void* a,
                         const void* a_scales, const void* bias, void* out, void* workspace, size_t ws_bytes,
                         const hum_tile_config* cfg, void* stream) {
  clear_error();
  Layout L;
  hum_status st = compute_layout(desc, &L);
  if (st != HUM_OK) return st;
  if (desc->num_experts != 1) return set_error(HUM_ERR_INVALID_ARG, "hum_linear takes a dense (num_experts == 1) description");
  if (m < 0) return set_error(HUM_ERR_INVALID_ARG, "m < 0");
  if (m == 0) return HUM_OK;
  if (!packed || !a || !out) return set_error(HUM_ERR_INVALID_ARG, "packed, a and out must be non-NULL");
  const bool quant_a = desc->act_fmt != HUM_ACT_BF16 && a_scales == nullptr;
  // (pre-quantized W4A4 activations are E2M1 codes: the tile kernels take them)
  hum_tile_config c = cfg ? *cfg : select_dense(desc, m, quant_a);
  if (!cfg_sane(c) || !gemm_instance_exists(dense_key(desc, c)) ||
      (c.split_k > 1 && !reduce_instance_exists(fmt_of(desc), EPI_BF16)))
    return set_error(HUM_ERR_UNSUPPORTED, "tile config not available");
  if (c.kind == HUM_KERNEL_STREAM && m > 16) return set_error(HUM_ERR_UNSUPPORTED, "the stream kernel takes m <= 16");
  if (w4a4_on_stream(desc, c) && !quant_a)
    return set_error(HUM_ERR_UNSUPPORTED, "W4A4 on the decode kernel quantizes its activations itself");
  // block-scaled FP8 on the decode kernel: the kernel quantizes the bf16 rows
  const bool blk_stream = fmt_of(desc) == F_FP8_BLOCK && c.kind == HUM_KERNEL_STREAM;
  if (blk_stream && !quant_a)
    return set_error(HUM_ERR_UNSUPPORTED, "block-scaled FP8 on the decode kernel quantizes its activations itself");
  const DenseWs w = dense_ws(desc, m, c, quant_a);
  if (w.total > 0 && (!workspace || ws_bytes < (size_t)w.total))
    return set_error(HUM_ERR_WORKSPACE, "workspace too small (%zu < %lld)", ws_bytes, (long long)w.total);
  log_cfg("linear", c, m);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const void* a_use = a;
  const void* as_use = a_scales;
  // Per-token FP8 activations on the dense decode kernel without split-K:
  // the kernel quantizes the bf16 rows itself (same codes and scales as the
  // quantizer launch, which it saves)
  const bool fuse_q = quant_a && desc->act_fmt == HUM_ACT_FP8_TOKEN && fmt_of(desc) == F_FP8 &&
                      c.kind == HUM_KERNEL_STREAM && c.split_k == 1 &&
                      stream_fp8_fuse_fits((int)m, kb_per_split(L.kb, c), c.waves_k);
  if (w4a4_on_stream(desc, c)) {
    st = launch_quant_mxfp4_wide(m, desc->k, a, desc->k, ws + w.aq, reinterpret_cast<uint8_t*>(ws + w.as), stream);
    if (st != HUM_OK) return st;
    a_use = ws + w.aq;
    as_use = ws + w.as;
  } else if (quant_a && !fuse_q && !blk_stream) {
    st = hum_quant_act(desc->act_fmt, m, desc->k, a, desc->k, ws + w.aq, ws + w.as, stream);
    if (st != HUM_OK) return st;
    a_use = ws + w.aq;
    as_use = ws + w.as;
  }
  GemmParams p{};
  fill_weight_params(p, desc, L, packed);
  if (fmt_int(fmt_of(desc)) && c.kind != HUM_KERNEL_STREAM) {
    st = launch_rowsum(a_use, desc->k, m, (int)L.kb, (int)L.kbc, ws + w.rowsum, stream);
    if (st != HUM_OK) return st;
    p.a_rowsum = ws + w.rowsum;
  }
  p.a = a_use;
  p.lda = desc->k;
  p.a_scale = as_use;
  // bytes per row of activation scales: E8M0 per 32, or f32 per 128
  p.a_scale_ld = desc->act_fmt == HUM_ACT_FP8_GROUP ? (desc->k / 128) * 4 : desc->k / 32;
  p.m = m;
  p.sorted = nullptr;
  p.block_expert = nullptr;
  p.live_rows = nullptr;
  p.topk = 1;
  p.sentinel = 0;
  p.out = out;
  p.ldo = desc->n;
  p.out_scale = nullptr;
  p.bias = static_cast<const uint16_t*>(bias);
  const int64_t m_tiles = cdiv(m, tile_rows(c));
  p.n_tiles = (int)cdiv(L.nt, tile_subtiles(c));
  p.group_m = 8;  // 8 M-tiles x all N-tiles share one XCD's L2
  p.split_k = c.split_k;
  p.kb_per_split = kb_per_split(L.kb, c);
  p.partials = reinterpret_cast<float*>(ws + w.partials);
  if (c.stream_k > 0) {
    const int64_t tiles = m_tiles * p.n_tiles;
    if (tiles > kSkMaxTiles) return set_error(HUM_ERR_UNSUPPORTED, "Stream-K takes at most %lld tiles", (long long)kSkMaxTiles);
    p.sk_tiles = (int)tiles;
    p.sk_m_tiles = (int)m_tiles;
    p.sk_len = cdiv(tiles * L.kb, c.stream_k);
    // workgroups that get iterations (the rest would have none)
    p.sk_groups = (int)cdiv(tiles * L.kb, p.sk_len);
    p.sk_count = reinterpret_cast<uint32_t*>(ws);
    p.sk_part = reinterpret_cast<float*>(ws + w.partials);
    p.sk_part_bytes = 2 * (int64_t)p.sk_groups * tile_rows(c) * tile_subtiles(c) * 16 * 4;
    if (p.sk_part_bytes >= ((int64_t)1 << 31)) return set_error(HUM_ERR_UNSUPPORTED, "Stream-K partial slots above 2 GiB");
  }
  p.stream_rows = (int)(m < 16 ? m : 16);
  p.a_bytes = (fmt_of(desc) == F_MXFP4_MXFP4 && !w4a4_on_stream(desc, c)) ? m * (desc->k / 2)
                                            : m * desc->k * ((fmt_bf16_act(fmt_of(desc)) || fuse_q || blk_stream) ? 2 : 1);
  p.a_fp8_fuse = fuse_q ? 1 : 0;
  p.a_scale_bytes = (desc->act_fmt == HUM_ACT_MXFP8 || desc->act_fmt == HUM_ACT_MXFP4) ? m * (desc->k / 32)
                    : (desc->act_fmt == HUM_ACT_FP8_GROUP ? m * (desc->k / 128) * 4 : 0);
  return launch_gemm(dense_key(desc, c), p, m_tiles, (int)tile_rows(c), stream);
}

hum_status hum_linear(const hum_weight_desc* desc, const void* packed, int64_t m, const void* a, const void* a_scales,
                      const void* bias, void* out, void* workspace, size_t ws_bytes, void* stream) {
  return hum_linear_ex(desc, packed, m, a, a_scales, bias, out, workspace, ws_bytes, nullptr, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// No-allocation variant of hum_linear: its workspace (split-K partials,
// quantized activations, row sums) lives in this fixed static device array.
// Each GPU the library runs on holds its own copy until the process ends.
// In host code the array's name is only a stand-in: its device address is
// looked up once per device (with that device current) and kept.

namespace hum {
static __device__ __align__(256) uint8_t scratch[HUM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static void* g_scratch_dev[kMaxDevices];
static std::mutex g_scratch_mu;

// Device address of this device's scratch array (looked up on first use).
static hum_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return set_error(HUM_ERR_HIP, "hipGetDevice failed");
  if (dev >= kMaxDevices) return set_error(HUM_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(HUM_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return HUM_OK;
}
}  // namespace hum

extern "C" {

hum_status hum_linear_noalloc(const hum_weight_desc* desc, const void* packed, int64_t m, const void* a,
                              const void* a_scales, const void* bias, void* out, void* stream) {
  clear_error();
  hum_status st = check_desc(desc);
  if (st != HUM_OK) return st;
  if (m < 0) return set_error(HUM_ERR_INVALID_ARG, "m < 0");
  if (m == 0) return HUM_OK;
  const bool quant_a = desc->act_fmt != HUM_ACT_BF16 && a_scales == nullptr;
  const hum_tile_config c = select_dense(desc, m, quant_a);
  const int64_t need = dense_ws(desc, m, c, quant_a).total;
  if (need > (int64_t)HUM_NOALLOC_SCRATCH_BYTES)
    return set_error(HUM_ERR_WORKSPACE,
                     "hum_linear_noalloc: this call needs %lld bytes of scratch; the static array holds %lld "
                     "(use hum_linear with a workspace)",
                     (long long)need, (long long)HUM_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != HUM_OK) return st;
  return hum_linear_ex(desc, packed, m, a, a_scales, bias, out, ws, (size_t)HUM_NOALLOC_SCRATCH_BYTES, &c, stream);
}

// ---------------------------------------------------------------------------
// On-device autotune: every compiled dense configuration, timed on the
// caller's own buffers.

static void dense_candidates(const hum_weight_desc* d, int64_t m, uint32_t flags, std::vector<hum_tile_config>& out) {
  const int64_t kb = d->k / kKBlk;
  const bool inv = (flags & HUM_SELECT_BATCH_INVARIANT) != 0;
  for (int split = 1; split <= 16; split *= 2) {
    if (inv && split > 1) break;
    for (int kind = HUM_KERNEL_TILE; kind <= HUM_KERNEL_TILE32; ++kind) {
      if (kind == HUM_KERNEL_STREAM && (inv || m > 16)) continue;
      if (kind == HUM_KERNEL_TILE32 && inv) continue;
      const bool tile = kind != HUM_KERNEL_STREAM;
      for (int wm = 1; wm <= (tile ? 8 : 1); wm *= 2)
        for (int wn = 1; wn <= 8; wn *= 2)
          for (int wk = 1; wk <= (tile ? 1 : 15); ++wk)
            for (int st = 0; st <= (tile ? 3 : 0); st += 3) {
              hum_tile_config c{};
              c.kind = kind;
              c.wave_m = wm;
              c.wave_n = wn;
              c.waves_n = tile ? 4 : 1;
              c.waves_k = wk;
              c.split_k = split;
              c.stages = st;
              c.block_m = (int32_t)tile_rows(c);
              // every split must own at least one K-block
              if (split > 1 && (int64_t)kb_per_split(kb, c) * (split - 1) >= kb) continue;
              if (cfg_sane(c) && gemm_instance_exists(dense_key(d, c))) out.push_back(c);
              // Stream-K over 256 / 512 / 1024 workgroups
              if (split == 1 && tile && !inv)
                for (int g = 256; g <= 1024; g *= 2) {
                  hum_tile_config k = c;
                  k.stream_k = g;
                  if (cdiv(m, tile_rows(k)) * cdiv(cdiv(d->n, kNSub), tile_subtiles(k)) <= kSkMaxTiles &&
                      cfg_sane(k) && gemm_instance_exists(dense_key(d, k)))
                    out.push_back(k);
                }
            }
    }
  }
}

hum_status hum_autotune_linear(const hum_weight_desc* desc, const void* packed, int64_t m, const void* a,
                               const void* a_scales, const void* bias, void* out, void* workspace, size_t ws_bytes,
                               int32_t iters, uint32_t flags, hum_tile_config* best_out, float* best_us_out,
                               void* stream) {
  clear_error();
  hum_status st = check_desc(desc);
  if (st != HUM_OK) return st;
  if (desc->num_experts != 1) return set_error(HUM_ERR_INVALID_ARG, "autotune takes a dense (num_experts == 1) description");
  if (m < 1 || iters < 1 || iters > 10000 || !best_out) return set_error(HUM_ERR_INVALID_ARG, "bad m / iters / best_out");
  if (flags & ~(uint32_t)HUM_SELECT_BATCH_INVARIANT) return set_error(HUM_ERR_INVALID_ARG, "unknown selection flags 0x%x", flags);
  if (!packed || !a || !out) return set_error(HUM_ERR_INVALID_ARG, "packed, a and out must be non-NULL");
  std::vector<hum_tile_config> cands;
  dense_candidates(desc, m, flags, cands);
  const bool quant_a = desc->act_fmt != HUM_ACT_BF16 && a_scales == nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return set_error(HUM_ERR_HIP, "hipEventCreate failed");
  }
  float best_us = 0.0f;
  hum_tile_config best{};
  bool found = false;
  for (const hum_tile_config& c : cands) {
    const int64_t need = dense_ws(desc, m, c, quant_a).total;
    if (need > 0 && (!workspace || (int64_t)ws_bytes < need)) continue;
    // one untimed call: warms the code object and screens configurations the
    // launcher refuses for this shape (the decode kernel's K-range limits)
    st = hum_linear_ex(desc, packed, m, a, a_scales, bias, out, workspace, ws_bytes, &c, stream);
    if (st == HUM_ERR_UNSUPPORTED) continue;
    if (st == HUM_OK && hipEventRecord(e0, s) != hipSuccess) st = set_error(HUM_ERR_HIP, "hipEventRecord failed");
    for (int i = 0; i < iters && st == HUM_OK; ++i)
      st = hum_linear_ex(desc, packed, m, a, a_scales, bias, out, workspace, ws_bytes, &c, stream);
    float ms = 0.0f;
    if (st == HUM_OK && (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                         hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
      st = set_error(HUM_ERR_HIP, "timing events failed");
    if (st != HUM_OK) {
      (void)hipEventDestroy(e0);
      (void)hipEventDestroy(e1);
      return st;
    }
    const float us = ms * 1000.0f / (float)iters;
    if (!found || us < best_us) {
      best_us = us;
      best = c;
      found = true;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (!found) return set_error(HUM_ERR_UNSUPPORTED, "no compiled configuration fits this shape and workspace");
  // leave the winner's result in out
  st = hum_linear_ex(desc, packed, m, a, a_scales, bias, out, workspace, ws_bytes, &best, stream);
  if (st != HUM_OK) return st;
  *best_out = best;
  if (best_us_out) *best_us_out = best_us;
  return HUM_OK;
}

// ---------------------------------------------------------------------------
// MoE.

// Bytes of `rows` activation rows of length k in activation format `fmt`:
// codes, and scales (MX: E8M0 per 32; FP8 per token: f32 per row; FP8 per
// group: f32 per 128).
struct ActBytes {
  int64_t codes, scales;
};
static ActBytes act_bytes(int fmt, int64_t rows, int64_t k) {
  switch (fmt) {
    case HUM_ACT_FP8_TOKEN: return {rows * k, rows * 4};
    case HUM_ACT_MXFP8: return {rows * k, rows * (k / 32)};
    case HUM_ACT_MXFP4: return {rows * (k / 2), rows * (k / 32)};
    case HUM_ACT_FP8_GROUP: return {rows * k, rows * (k / 128) * 4};
    default: return {rows * k * 2, 0};
  }
}
// Bytes per row of the activation scales the GEMM kernels stage per row.
static int64_t act_scale_ld(int fmt, int64_t k) {
  return fmt == HUM_ACT_FP8_GROUP ? (k / 128) * 4 : (fmt == HUM_ACT_FP8_TOKEN ? 4 : k / 32);
}
// The gate_up epilogue requantizes the SwiGLU output itself (MX formats) or
// writes it in bf16, to be quantized by a kernel between the GEMMs (FP8 per
// token / per group) or used as is (bf16).
static bool act_fused_requant(int fmt) { return fmt == HUM_ACT_MXFP8 || fmt == HUM_ACT_MXFP4; }
static bool act_separate_quant(int fmt) { return fmt == HUM_ACT_FP8_TOKEN || fmt == HUM_ACT_FP8_GROUP; }

struct MoeWs {
  int64_t partials = 0, sorted = 0, offsets = 0, counts = 0, bexp = 0, align_tmp = 0;
  int64_t xq = 0, xs = 0, inter = 0, inter_s = 0, interq = 0, interq_s = 0, y = 0, total = 0;
  int64_t cap = 0, nblocks = 0;
};

// masked: t rows of the [E][max_m] layout, one slot per row, slot = row
// (no padding beyond max_m, output written by the down GEMM in place).
static MoeWs moe_ws(const hum_weight_desc* w13, const hum_weight_desc* w2, int64_t t, int32_t topk,
                    const MoeCfg& mc, bool masked = false) {
  MoeWs w;
  const int64_t E = w13->num_experts;
  const int64_t bm = tile_rows(mc.up);
  const int split = mc.up.split_k > mc.dn.split_k ? mc.up.split_k : mc.dn.split_k;
  const int64_t inter = w2->k;
  const int64_t h = w13->k;
  const int act = w13->act_fmt;
  w.cap = masked ? t : t * topk + E * (bm - 1);
  w.nblocks = cdiv(w.cap, bm);
  const int64_t pcols = (2 * inter > cdiv(h, kNSub) * kNSub) ? 2 * inter : cdiv(h, kNSub) * kNSub;
  int64_t off = kWsHeader;  // (the Stream-K counters of dense calls sharing the workspace)
  w.partials = off;
  if (split > 1) off = align256(off + (int64_t)split * w.cap * pcols * 4);
  w.sorted = off;
  off = align256(off + w.cap * 4);
  w.offsets = off;
  off = align256(off + (E + 1) * 4);
  w.counts = off;
  off = align256(off + E * 4);
  w.bexp = off;
  off = align256(off + w.nblocks * 4);
  w.align_tmp = off;  // per-chunk expert counts of the multi-workgroup sort
  if (!masked) off = align256(off + align_workspace_bytes(t, topk, (int32_t)E));
  w.xq = off;
  if (act != HUM_ACT_BF16) {
    // (W4A4 gate_up on the decode kernel reads the codes as E4M3 bytes)
    const bool wide = act == HUM_ACT_MXFP4 && mc.up.kind == HUM_KERNEL_STREAM;
    const ActBytes ab = act_bytes(wide ? HUM_ACT_MXFP8 : act, t, h);
    off = align256(off + ab.codes);
    w.xs = off;
    off = align256(off + ab.scales);
  }
  // gate_up output: MX codes (+ scales) when requantized in the epilogue,
  // else bf16
  w.inter = off;
  const ActBytes ib = act_bytes(act_fused_requant(act) ? act : HUM_ACT_BF16, w.cap, inter);
  off = align256(off + ib.codes);
  w.inter_s = off;
  off = align256(off + ib.scales);
  // FP8 per token / per group: the intermediate quantized between the GEMMs
  w.interq = off;
  if (act_separate_quant(act)) {
    const ActBytes qb = act_bytes(act, w.cap, inter);
    off = align256(off + qb.codes);
    w.interq_s = off;
    off = align256(off + qb.scales);
  }
  w.y = off;
  if (!masked) off = align256(off + t * topk * h * 2);
  w.total = off;
  return w;
}

static hum_status check_moe(const hum_weight_desc* w13, const hum_weight_desc* w2, int64_t t, int32_t topk) {
  hum_status st = check_desc(w13);
  if (st != HUM_OK) return st;
  st = check_desc(w2);
  if (st != HUM_OK) return st;
  if (w13->num_experts != w2->num_experts) return set_error(HUM_ERR_INVALID_ARG, "w13 and w2 expert counts differ");
  if (w13->act_fmt != w2->act_fmt) return set_error(HUM_ERR_INVALID_ARG, "w13 and w2 activation formats differ");
  if (fmt_of(w13) != fmt_of(w2)) return set_error(HUM_ERR_INVALID_ARG, "w13 and w2 weight formats differ");
  if (!moe_fmt_ok(fmt_of(w13)))
    return set_error(HUM_ERR_UNSUPPORTED,
                     "the MoE path runs MXFP4, MXINT4, NVFP4, FP8 (per-channel / per-tensor / 128-block) and INT8 "
                     "expert weights; not INT4 / UINT4 with group scales");
  if (w13->n != 2 * w2->k) return set_error(HUM_ERR_INVALID_ARG, "w13 n must be 2 * intermediate (w2 k)");
  if (w2->n != w13->k) return set_error(HUM_ERR_INVALID_ARG, "w2 n must equal the hidden size (w13 k)");
  if (w2->k % 128) return set_error(HUM_ERR_UNSUPPORTED, "intermediate size must be a multiple of 128");
  if (t < 0 || topk < 1 || topk > 64) return set_error(HUM_ERR_INVALID_ARG, "bad num_tokens / topk");
  if (w13->num_experts > 512) return set_error(HUM_ERR_UNSUPPORTED, "at most 512 experts");
  if ((t * topk + (int64_t)w13->num_experts * 127) >= ((int64_t)1 << 31)) return set_error(HUM_ERR_UNSUPPORTED, "too many tokens");
  // activation buffers read through 32-bit buffer offsets
  if (t * w13->k * 2 >= ((int64_t)1 << 31) || (t * topk + (int64_t)w13->num_experts * 127) * w2->k * 2 >= ((int64_t)1 << 31))
    return set_error(HUM_ERR_UNSUPPORTED, "MoE activations above 2 GiB");
  return HUM_OK;
}

hum_status hum_moe_select_config(const hum_weight_desc* w13, const hum_weight_desc* w2, int64_t t, int32_t topk,
                                 uint32_t flags, hum_tile_config* cfg_out) {
  clear_error();
  hum_status st = check_moe(w13, w2, t, topk);
  if (st != HUM_OK) return st;
  if (!cfg_out) return set_error(HUM_ERR_INVALID_ARG, "cfg_out is NULL");
  if (flags & ~(uint32_t)(HUM_SELECT_BATCH_INVARIANT | HUM_SELECT_MOE_GATE_UP))
    return set_error(HUM_ERR_INVALID_ARG, "unknown selection flags 0x%x", flags);
  const MoeCfg mc = select_moe(w13, t < 1 ? 1 : t, topk, w2);
  hum_tile_config c = (flags & HUM_SELECT_MOE_GATE_UP) ? mc.up : mc.dn;
  // the grouped tile kernel sums each slot's row in a fixed order (no split-K);
  // the decode kernel splits K inside the workgroup.  The invariant layer runs
  // one configuration for both GEMMs: the 256-column tiles (the decode-size
  // down GEMM's 128-column tile has no gate_up instance)
  if ((flags & HUM_SELECT_BATCH_INVARIANT) && (c.kind != HUM_KERNEL_TILE || c.wave_n != 4))
    c = moe_tile_cfg(c.kind == HUM_KERNEL_TILE ? c.wave_m : 1);
  *cfg_out = c;
  return HUM_OK;
}

size_t hum_moe_workspace_bytes_ex(const hum_weight_desc* w13, const hum_weight_desc* w2, int64_t t, int32_t topk,
                                  const hum_tile_config* cfg) {
  clear_error();
  if (check_moe(w13, w2, t, topk) != HUM_OK) return 0;
  const MoeCfg mc = cfg ? MoeCfg{*cfg, *cfg} : select_moe(w13, t, topk, w2);
  return (size_t)moe_ws(w13, w2, t, topk, mc).total;
}

size_t hum_moe_workspace_bytes(const hum_weight_desc* w13, const hum_weight_desc* w2, int64_t t, int32_t topk) {
  return hum_moe_workspace_bytes_ex(w13, w2, t, topk, nullptr);
}

hum_status hum_moe_align(const int32_t* topk_ids, int64_t t, int32_t topk, int32_t e, int32_t block_m,
                         int32_t* sorted, int32_t* offsets, int32_t* counts, void* stream) {
  clear_error();
  if (t < 0 || topk < 1 || e < 1 || block_m < 1) return set_error(HUM_ERR_INVALID_ARG, "bad sizes");
  if (!sorted || !offsets || !counts || (t > 0 && !topk_ids)) return set_error(HUM_ERR_INVALID_ARG, "NULL pointer");
  if (e > 512) return set_error(HUM_ERR_UNSUPPORTED, "at most 512 experts");
  // The block -> expert map the GEMMs use is internal; this export skips it.
  return launch_align(topk_ids, t, topk, e, block_m, sorted, offsets, counts, nullptr, 0, stream);
}

size_t hum_moe_align_workspace_bytes(int64_t t, int32_t topk, int32_t e) {
  clear_error();
  if (t < 0 || topk < 1 || e < 1) return 0;
  return (size_t)align_workspace_bytes(t, topk, e);
}

hum_status hum_moe_align_ex(const int32_t* topk_ids, int64_t t, int32_t topk, int32_t e, int32_t block_m,
                            int32_t* sorted, int32_t* offsets, int32_t* counts, void* workspace, size_t ws_bytes,
                            void* stream) {
  clear_error();
  if (t < 0 || topk < 1 || e < 1 || block_m < 1) return set_error(HUM_ERR_INVALID_ARG, "bad sizes");
  if (!sorted || !offsets || !counts || (t > 0 && !topk_ids)) return set_error(HUM_ERR_INVALID_ARG, "NULL pointer");
  if (e > 512) return set_error(HUM_ERR_UNSUPPORTED, "at most 512 experts");
  const int64_t need = align_workspace_bytes(t, topk, e);
  if (need > 0 && (!workspace || (int64_t)ws_bytes < need))
    return set_error(HUM_ERR_WORKSPACE, "workspace too small (%zu < %lld)", ws_bytes, (long long)need);
  return launch_align(topk_ids, t, topk, e, block_m, sorted, offsets, counts, nullptr, 0, stream, workspace,
                      (int64_t)ws_bytes);
}

hum_status hum_moe_reduce(const void* y_bf16, const float* topk_weights, int64_t t, int32_t topk, int64_t h,
                          void* out_bf16, void* stream) {
  clear_error();
  if (t < 0 || topk < 1 || h < 8 || h % 8) return set_error(HUM_ERR_INVALID_ARG, "bad sizes (h must be a multiple of 8)");
  if (t > 0 && (!y_bf16 || !topk_weights || !out_bf16)) return set_error(HUM_ERR_INVALID_ARG, "NULL pointer");
  return launch_moe_reduce(y_bf16, topk_weights, t, topk, h, out_bf16, stream);
}

// ---- one grouped GEMM (stage export) -------------------------------------

struct StageSetup {
  hum_tile_config c;
  KernelKey key;
  int64_t nblocks = 0, bexp = 0, partials = 0, total = 0;
};

static int stage_epi(int32_t e) {
  switch (e) {
    case HUM_MOE_EPI_NONE: return EPI_BF16;
    case HUM_MOE_EPI_SCATTER: return EPI_SCATTER;
    case HUM_MOE_EPI_SWIGLU_BF16: return EPI_SWIGLU_BF16;
    case HUM_MOE_EPI_SWIGLU_MXFP8: return EPI_SWIGLU_MXFP8;
    case HUM_MOE_EPI_SWIGLU_MXFP4: return EPI_SWIGLU_MXFP4;
  }
  return -1;
}

// Validation, configuration and workspace plan of hum_moe_grouped_gemm.
static hum_status stage_setup(const hum_weight_desc* w, int32_t a_mode, int32_t epilogue, int64_t t, int32_t topk,
                              int64_t sorted_len, int32_t block_m, const hum_tile_config* cfg, StageSetup* out) {
  hum_status st = check_desc(w);
  if (st != HUM_OK) return st;
  const int f = fmt_of(w);
  if (!moe_fmt_ok(f)) return set_error(HUM_ERR_UNSUPPORTED, "no grouped GEMM for this weight format");
  if (w->num_experts > 512) return set_error(HUM_ERR_UNSUPPORTED, "at most 512 experts");
  if (t < 0 || topk < 1 || topk > 64 || sorted_len < 0) return set_error(HUM_ERR_INVALID_ARG, "bad num_tokens / topk / sorted_len");
  if (block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128)
    return set_error(HUM_ERR_INVALID_ARG, "block_m must be 16, 32, 64 or 128");
  if (a_mode != HUM_MOE_A_GATHER && a_mode != HUM_MOE_A_SORTED) return set_error(HUM_ERR_INVALID_ARG, "bad a_mode");
  const int epi = stage_epi(epilogue);
  if (epi < 0) return set_error(HUM_ERR_INVALID_ARG, "bad epilogue");
  const bool swiglu = epi == EPI_SWIGLU_BF16 || epi == EPI_SWIGLU_MXFP8 || epi == EPI_SWIGLU_MXFP4;
  if (swiglu && w->n % 64) return set_error(HUM_ERR_INVALID_ARG, "SwiGLU epilogues need n = 2 * I with I % 32 == 0");
  if (swiglu && epi != moe_up_epi(f))
    return set_error(HUM_ERR_UNSUPPORTED, "this activation format's SwiGLU epilogue is %s",
                     moe_up_epi(f) == EPI_SWIGLU_MXFP8 ? "SWIGLU_MXFP8"
                                                      : (moe_up_epi(f) == EPI_SWIGLU_MXFP4 ? "SWIGLU_MXFP4" : "SWIGLU_BF16"));
  if (t * topk + (int64_t)w->num_experts * 127 >= ((int64_t)1 << 31) || sorted_len >= ((int64_t)1 << 31))
    return set_error(HUM_ERR_UNSUPPORTED, "too many rows");
  StageSetup S;
  if (cfg) {
    S.c = *cfg;
  } else {
    const MoeCfg mc = select_moe_shape(w, t < 1 ? 1 : t, topk);
    S.c = (tile_rows(mc.dn) == block_m) ? mc.dn : moe_tile_cfg(block_m / 16);
  }
  if (!cfg_sane(S.c) || S.c.stream_k != 0) return set_error(HUM_ERR_UNSUPPORTED, "tile config not available");
  if (tile_rows(S.c) != block_m) return set_error(HUM_ERR_INVALID_ARG, "the configuration's block (%d rows) differs from block_m", (int)tile_rows(S.c));
  // sorted rows: the scatter epilogue's instances read them directly (that
  // epilogue implies grouped rows); the others take the grouped-row mode
  const int amode = a_mode == HUM_MOE_A_GATHER ? A_GATHER : (epi == EPI_SCATTER ? A_DIRECT : A_SORTED);
  S.key = KernelKey{f, S.c.kind, S.c.wave_m, S.c.wave_n, S.c.waves_n, S.c.waves_k, amode, epi, key_stages(S.c)};
  if (!cfg && S.c.stages == 3 && !gemm_instance_exists(S.key)) {
    // the layer's three-stage tiles exist for its own modes only
    S.c.stages = 0;
    S.key.stages = key_stages(S.c);
  }
  if (!gemm_instance_exists(S.key)) return set_error(HUM_ERR_UNSUPPORTED, "no grouped GEMM instance for this mode, epilogue and tile");
  if (S.c.split_k > 1 && !reduce_instance_exists(f, epi)) return set_error(HUM_ERR_UNSUPPORTED, "no split-K reduce for this format and epilogue");
  if (S.c.kind == HUM_KERNEL_STREAM && !moe_stream_fits(w, S.c, (int)(t * topk < 16 ? t * topk : 16)))
    return set_error(HUM_ERR_UNSUPPORTED, "decode kernel: K range per split too long for LDS (raise split_k)");
  S.nblocks = cdiv(sorted_len, block_m);
  int64_t off = kWsHeader;  // (the Stream-K counters of dense calls sharing the workspace)
  S.bexp = off;
  off = align256(off + S.nblocks * 4);
  S.partials = off;
  const int64_t ncols = swiglu ? w->n : cdiv(w->n, kNSub) * kNSub;
  if (S.c.split_k > 1) off = align256(off + (int64_t)S.c.split_k * sorted_len * ncols * 4);
  S.total = off;
  *out = S;
  return HUM_OK;
}

size_t hum_moe_grouped_gemm_workspace_bytes(const hum_weight_desc* w, int32_t a_mode, int32_t epilogue,
                                            int64_t num_tokens, int32_t topk, int64_t sorted_len, int32_t block_m,
                                            const hum_tile_config* cfg) {
  clear_error();
  StageSetup S;
  if (stage_setup(w, a_mode, epilogue, num_tokens, topk, sorted_len, block_m, cfg, &S) != HUM_OK) return 0;
  return (size_t)(S.total > 0 ? S.total : 256);
}

hum_status hum_moe_grouped_gemm(const hum_weight_desc* w, const void* packed, int32_t a_mode, int32_t epilogue,
                                int64_t num_tokens, int32_t topk, const void* a, const void* a_scales,
                                const int32_t* sorted, int64_t sorted_len, const int32_t* offsets, int32_t block_m,
                                void* out, void* out_scales, float* out_swiglu_f32, const hum_tile_config* cfg,
                                void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  StageSetup S;
  hum_status st = stage_setup(w, a_mode, epilogue, num_tokens, topk, sorted_len, block_m, cfg, &S);
  if (st != HUM_OK) return st;
  if (sorted_len == 0 || num_tokens == 0) return HUM_OK;
  const int act = w->act_fmt;
  const int epi = stage_epi(epilogue);
  const bool swiglu = epi == EPI_SWIGLU_BF16 || epi == EPI_SWIGLU_MXFP8 || epi == EPI_SWIGLU_MXFP4;
  if (!packed || !a || !sorted || !offsets || !out) return set_error(HUM_ERR_INVALID_ARG, "NULL pointer");
  if (act != HUM_ACT_BF16 && !a_scales) return set_error(HUM_ERR_INVALID_ARG, "quantized activations need a_scales");
  if ((epi == EPI_SWIGLU_MXFP8 || epi == EPI_SWIGLU_MXFP4) && !out_scales)
    return set_error(HUM_ERR_INVALID_ARG, "MX epilogues need out_scales");
  if (!workspace || ws_bytes < (size_t)S.total)
    return set_error(HUM_ERR_WORKSPACE, "workspace too small (%zu < %lld)", ws_bytes, (long long)S.total);
  const int64_t a_rows = a_mode == HUM_MOE_A_GATHER ? num_tokens : sorted_len;
  const ActBytes ab = act_bytes(act, a_rows, w->k);
  if (ab.codes >= ((int64_t)1 << 31) || ab.scales >= ((int64_t)1 << 31))
    return set_error(HUM_ERR_UNSUPPORTED, "activations above 2 GiB");
  Layout L;
  compute_layout(w, &L);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* bexp = reinterpret_cast<int32_t*>(ws + S.bexp);
  st = launch_block_expert(offsets, w->num_experts, block_m, S.nblocks, bexp, stream);
  if (st != HUM_OK) return st;
  GemmParams p{};
  fill_weight_params(p, w, L, packed);
  const int64_t nout = swiglu ? w->n / 2 : w->n;
  p.n = nout;
  p.swiglu_nt_off = swiglu ? (int)(nout / kNSub) : 0;
  p.a = a;
  p.lda = w->k;
  p.a_scale = a_scales;
  p.a_scale_ld = act_scale_ld(act, w->k);
  p.m = sorted_len;
  p.sorted = sorted;
  p.block_expert = bexp;
  p.live_rows = offsets + w->num_experts;
  p.topk = topk;
  p.sentinel = (int)(num_tokens * topk);
  p.out = out;
  p.ldo = nout;
  p.out_scale = out_scales;
  p.swiglu_f32 = swiglu ? out_swiglu_f32 : nullptr;
  p.bias = nullptr;
  p.n_tiles = (int)(swiglu ? cdiv(cdiv(nout, kNSub), tile_subtiles(S.c) / 2) : cdiv(L.nt, tile_subtiles(S.c)));
  p.group_m = 1;  // M-tiles are different experts
  p.split_k = S.c.split_k;
  p.kb_per_split = kb_per_split(L.kb, S.c);
  p.partials = reinterpret_cast<float*>(ws + S.partials);
  p.stream_rows = (int)(num_tokens * topk < 16 ? num_tokens * topk : 16);
  p.a_bytes = ab.codes;
  p.a_scale_bytes = ab.scales;
  log_cfg("moe grouped gemm", S.c, sorted_len);
  return launch_gemm(S.key, p, S.nblocks, block_m, stream);
}

// Kernel keys of a layer's two GEMMs; HUM_OK when both are compiled.
static hum_status moe_keys(const hum_weight_desc* w13, const MoeCfg& mc, KernelKey* kup, KernelKey* kdn) {
  const hum_tile_config& cu = mc.up;
  const hum_tile_config& cd = mc.dn;
  if (!cfg_sane(cu) || !cfg_sane(cd) || cu.stream_k != 0 || cd.stream_k != 0 || tile_rows(cu) != tile_rows(cd))
    return set_error(HUM_ERR_UNSUPPORTED, "tile config not available");
  const int f = fmt_of(w13);
  const int epi_up = moe_up_epi(f);
  const int fu = cu.kind == HUM_KERNEL_STREAM ? moe_stream_fmt(f) : f;
  *kup = KernelKey{fu, cu.kind, cu.wave_m, cu.wave_n, cu.waves_n, cu.waves_k, A_GATHER, epi_up, key_stages(cu)};
  *kdn = KernelKey{f, cd.kind, cd.wave_m, cd.wave_n, cd.waves_n, cd.waves_k, A_DIRECT, EPI_SCATTER, key_stages(cd)};
  if (!gemm_instance_exists(*kup) || !gemm_instance_exists(*kdn)) return set_error(HUM_ERR_UNSUPPORTED, "tile config not available");
  if ((cu.split_k > 1 && !reduce_instance_exists(f, epi_up)) || (cd.split_k > 1 && !reduce_instance_exists(f, EPI_SCATTER)))
    return set_error(HUM_ERR_UNSUPPORTED, "no split-K reduce for this MoE format");
  return HUM_OK;
}

// The rows of one expert layer call, as the two GEMMs see them.
struct MoeRows {
  int64_t x_rows;         // rows of x (activations quantized before gate_up)
  int32_t topk;           // a sorted slot f reads x row f / topk
  int32_t sentinel;       // slots >= sentinel are padding
  int32_t stream_rows;    // upper bound of the valid rows of one expert block
  const int32_t* counts;  // grouped_masked: live rows per expert buffer (else NULL)
  int64_t max_m;          // grouped_masked: rows per expert buffer
  // indexed layout at decode sizes: the gate_up decode kernel routes the
  // slots itself (no align launch) and writes the arrays the down GEMM reads
  const int32_t* route_ids = nullptr;
  int32_t route_e = 0;
};

// gate_up (+ SwiGLU, + requantization) into the workspace, then down with
// its rows scattered to y[slot] (row stride h), over the expert blocks that
// ws.sorted / ws.bexp describe.  The layer input is quantized first where
// the activation format asks for it; FP8 per-token / per-group layers also
// quantize the bf16 SwiGLU output (its live rows) before the down GEMM.
static hum_status moe_gemms(const hum_weight_desc* w13, const void* packed_w13, const hum_weight_desc* w2,
                            const void* packed_w2, const MoeCfg& mc, const KernelKey& kup, const KernelKey& kdn,
                            const MoeWs& w, uint8_t* ws, const MoeRows& r, const void* x_bf16, void* y,
                            void* stream) {
  Layout L13, L2;
  compute_layout(w13, &L13);
  compute_layout(w2, &L2);
  const int64_t h = w13->k, inter = w2->k, t = r.x_rows;
  const hum_tile_config& cu = mc.up;
  const hum_tile_config& cd = mc.dn;
  const int32_t bm = (int32_t)tile_rows(cu);
  // Row tiles to launch.  Indexed layout: an expert with rows fills whole
  // blocks from its (block-aligned) segment start, so the live blocks are a
  // prefix of the padded block array, at most one per routed slot -- the
  // blocks past t * topk are all padding and are not launched (at decode
  // sizes most of the E * (block_m - 1) padding would be).  Masked layout:
  // every expert buffer's blocks.
  const int64_t m_tiles = r.counts ? w.nblocks : std::min<int64_t>(w.nblocks, t * (int64_t)r.topk);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + w.sorted);
  int32_t* bexp = reinterpret_cast<int32_t*>(ws + w.bexp);
  const int act = w13->act_fmt;
  const bool fused_q = act_fused_requant(act);
  const bool sep_q = act_separate_quant(act);
  const void* x_use = x_bf16;
  hum_status st = HUM_OK;
  // W4A4 gate_up on the decode kernel: MXFP4 codes as E4M3 bytes
  const bool wide_a = act == HUM_ACT_MXFP4 && kup.kind == KIND_STREAM;
  if (wide_a) {
    st = launch_quant_mxfp4_wide(t, h, x_bf16, h, ws + w.xq, ws + w.xs, stream);
  } else if (act == HUM_ACT_MXFP4) {
    st = launch_quant_mxfp4(t, h, x_bf16, h, ws + w.xq, ws + w.xs, stream, r.counts, r.max_m);
  } else if (act == HUM_ACT_MXFP8) {
    st = launch_quant_mxfp8(t, h, x_bf16, h, ws + w.xq, ws + w.xs, stream, r.counts, r.max_m);
  } else if (act == HUM_ACT_FP8_TOKEN) {
    st = launch_quant_fp8_token(t, h, x_bf16, h, ws + w.xq, reinterpret_cast<float*>(ws + w.xs), stream);
  } else if (act == HUM_ACT_FP8_GROUP) {
    st = launch_quant_fp8_group(t, h, x_bf16, h, ws + w.xq, reinterpret_cast<float*>(ws + w.xs), stream);
  }
  if (st != HUM_OK) return st;
  if (act != HUM_ACT_BF16) x_use = ws + w.xq;
  // gate_up (+ SwiGLU)
  GemmParams p{};
  fill_weight_params(p, w13, L13, packed_w13);
  p.n = inter;
  p.swiglu_nt_off = (int)(inter / kNSub);
  p.a = x_use;
  p.lda = h;
  p.a_scale = act != HUM_ACT_BF16 ? ws + w.xs : nullptr;
  p.a_scale_ld = act_scale_ld(act, h);
  p.m = w.cap;
  p.sorted = sorted;
  p.block_expert = bexp;
  p.live_rows = r.counts ? nullptr : reinterpret_cast<const int32_t*>(ws + w.offsets) + w13->num_experts;
  p.group_m = 1;  // N fastest over each expert block (groups of 8 blocks, M fastest, measured 0-10% slower)
  p.topk = r.topk;
  p.sentinel = r.sentinel;
  p.out = ws + w.inter;
  p.ldo = inter;
  p.out_scale = fused_q ? ws + w.inter_s : nullptr;
  p.bias = nullptr;
  p.n_tiles = (int)cdiv(cdiv(inter, kNSub), tile_subtiles(cu) / 2);
  p.split_k = cu.split_k;
  p.kb_per_split = kb_per_split(L13.kb, cu);
  p.partials = reinterpret_cast<float*>(ws + w.partials);
  p.stream_rows = r.stream_rows;
  const ActBytes xb = act_bytes(wide_a ? HUM_ACT_MXFP8 : act, t, h);
  p.a_bytes = xb.codes;
  p.a_scale_bytes = xb.scales;
  if (r.route_ids) {
    p.route_ids = r.route_ids;
    p.route_n = r.sentinel;
    p.route_e = r.route_e;
    p.route_sorted = sorted;
    p.route_bexp = bexp;
    p.route_live = reinterpret_cast<int32_t*>(ws + w.offsets) + w13->num_experts;
  }
  st = launch_gemm(kup, p, m_tiles, bm, stream);
  if (st != HUM_OK) return st;
  // FP8 per token / per group: quantize the live rows of the intermediate
  const void* a2 = ws + w.inter;
  const void* s2 = fused_q ? ws + w.inter_s : nullptr;
  if (sep_q) {
    st = act == HUM_ACT_FP8_TOKEN
             ? launch_quant_fp8_token(w.cap, inter, ws + w.inter, inter, ws + w.interq,
                                      reinterpret_cast<float*>(ws + w.interq_s), stream, sorted, r.sentinel)
             : launch_quant_fp8_group(w.cap, inter, ws + w.inter, inter, ws + w.interq,
                                      reinterpret_cast<float*>(ws + w.interq_s), stream, sorted, r.sentinel);
    if (st != HUM_OK) return st;
    a2 = ws + w.interq;
    s2 = ws + w.interq_s;
  }
  // down (rows scattered back to flat slots)
  GemmParams q{};
  fill_weight_params(q, w2, L2, packed_w2);
  q.a = a2;
  q.lda = inter;
  q.a_scale = s2;
  q.a_scale_ld = act_scale_ld(act, inter);
  q.m = w.cap;
  q.sorted = sorted;
  q.block_expert = bexp;
  q.live_rows = p.live_rows;
  q.group_m = p.group_m;
  q.topk = r.topk;
  q.sentinel = r.sentinel;
  q.out = y;
  q.ldo = h;
  q.out_scale = nullptr;
  q.bias = nullptr;
  q.n_tiles = (int)cdiv(L2.nt, tile_subtiles(cd));
  q.split_k = cd.split_k;
  q.kb_per_split = kb_per_split(L2.kb, cd);
  q.partials = reinterpret_cast<float*>(ws + w.partials);
  q.stream_rows = r.stream_rows;  // valid (non-padding) rows of a block
  const ActBytes ab = act_bytes(act, w.cap, inter);
  q.a_bytes = ab.codes;
  q.a_scale_bytes = ab.scales;
  return launch_gemm(kdn, q, m_tiles, bm, stream);
}

hum_status hum_moe_gemm_ex(const hum_weight_desc* w13, const void* packed_w13, const hum_weight_desc* w2,
                           const void* packed_w2, int64_t t, int32_t topk, const void* x_bf16,
                           const int32_t* topk_ids, const float* topk_weights, void* out_bf16, void* workspace,
                           size_t ws_bytes, const hum_tile_config* cfg, void* stream) {
  clear_error();
  hum_status st = check_moe(w13, w2, t, topk);
  if (st != HUM_OK) return st;
  if (t == 0) return HUM_OK;
  if (!packed_w13 || !packed_w2 || !x_bf16 || !topk_ids || !topk_weights || !out_bf16)
    return set_error(HUM_ERR_INVALID_ARG, "NULL pointer");
  const MoeCfg mc = cfg ? MoeCfg{*cfg, *cfg} : select_moe(w13, t, topk, w2);
  KernelKey kup, kdn;
  st = moe_keys(w13, mc, &kup, &kdn);
  if (st != HUM_OK) return st;
  const MoeWs w = moe_ws(w13, w2, t, topk, mc);
  if (!workspace || ws_bytes < (size_t)w.total)
    return set_error(HUM_ERR_WORKSPACE, "workspace too small (%zu < %lld)", ws_bytes, (long long)w.total);
  log_cfg("moe up", mc.up, t);
  log_cfg("moe down", mc.dn, t);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int64_t E = w13->num_experts, h = w13->k;
  const int64_t slots = t * topk;
  // At most 64 routed slots with a single-pass gate_up decode kernel (16-row
  // blocks, no split-K on either GEMM, no separate requantization of the
  // intermediate): the gate_up kernel routes them itself, in the align's
  // order, and leaves the rows of every launched block for the down GEMM,
  // which saves the align launch.
  const bool route = slots <= 64 && mc.up.kind == HUM_KERNEL_STREAM && tile_rows(mc.up) == 16 &&
                     mc.up.split_k == 1 && mc.dn.split_k == 1 && !act_separate_quant(w13->act_fmt);
  if (!route) {
    st = launch_align(topk_ids, t, topk, (int32_t)E, (int32_t)tile_rows(mc.up), reinterpret_cast<int32_t*>(ws + w.sorted),
                      reinterpret_cast<int32_t*>(ws + w.offsets), reinterpret_cast<int32_t*>(ws + w.counts),
                      reinterpret_cast<int32_t*>(ws + w.bexp), w.nblocks, stream, ws + w.align_tmp,
                      align_workspace_bytes(t, topk, (int32_t)E));
    if (st != HUM_OK) return st;
  }
  MoeRows rows{t, topk, (int32_t)slots, (int32_t)(slots < 16 ? slots : 16), nullptr, 0};
  if (route) {
    rows.route_ids = topk_ids;
    rows.route_e = (int32_t)E;
  }
  st = moe_gemms(w13, packed_w13, w2, packed_w2, mc, kup, kdn, w, ws, rows, x_bf16, ws + w.y, stream);
  if (st != HUM_OK) return st;
  return launch_moe_reduce(ws + w.y, topk_weights, t, topk, h, out_bf16, stream, topk_ids, (int32_t)E);
}

// ---- on-device autotune of the MoE layer ---------------------------------------

static void moe_candidates(const hum_weight_desc* w13, uint32_t flags, std::vector<hum_tile_config>& out) {
  const bool inv = (flags & HUM_SELECT_BATCH_INVARIANT) != 0;
  for (int kind = HUM_KERNEL_TILE; kind <= HUM_KERNEL_STREAM; ++kind) {
    if (inv && kind == HUM_KERNEL_STREAM) continue;
    for (int wm = 1; wm <= (kind == HUM_KERNEL_TILE ? 8 : 1); wm *= 2)
      for (int wn = 1; wn <= 8; wn *= 2)
        for (int wk = 1; wk <= (kind == HUM_KERNEL_TILE ? 1 : 15); ++wk)
          for (int st = 0; st <= (kind == HUM_KERNEL_TILE ? 3 : 0); st += 3) {
            hum_tile_config c{};
            c.kind = kind;
            c.wave_m = wm;
            c.wave_n = wn;
            c.waves_n = kind == HUM_KERNEL_TILE ? 4 : 1;
            c.waves_k = wk;
            c.split_k = 1;
            c.stages = st;
            c.block_m = (int32_t)tile_rows(c);
            KernelKey kup, kdn;
            if (cfg_sane(c) && moe_keys(w13, MoeCfg{c, c}, &kup, &kdn) == HUM_OK) out.push_back(c);
          }
  }
  clear_error();
}

hum_status hum_autotune_moe(const hum_weight_desc* w13, const void* packed_w13, const hum_weight_desc* w2,
                            const void* packed_w2, int64_t t, int32_t topk, const void* x_bf16,
                            const int32_t* topk_ids, const float* topk_weights, void* out_bf16, void* workspace,
                            size_t ws_bytes, int32_t iters, uint32_t flags, hum_tile_config* best_out,
                            float* best_us_out, void* stream) {
  clear_error();
  hum_status st = check_moe(w13, w2, t, topk);
  if (st != HUM_OK) return st;
  if (t < 1 || iters < 1 || iters > 10000 || !best_out) return set_error(HUM_ERR_INVALID_ARG, "bad t / iters / best_out");
  if (flags & ~(uint32_t)HUM_SELECT_BATCH_INVARIANT) return set_error(HUM_ERR_INVALID_ARG, "unknown selection flags 0x%x", flags);
  if (!packed_w13 || !packed_w2 || !x_bf16 || !topk_ids || !topk_weights || !out_bf16)
    return set_error(HUM_ERR_INVALID_ARG, "NULL pointer");
  std::vector<hum_tile_config> cands;
  moe_candidates(w13, flags, cands);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return set_error(HUM_ERR_HIP, "hipEventCreate failed");
  }
  float best_us = 0.0f;
  hum_tile_config best{};
  bool found = false;
  for (const hum_tile_config& c : cands) {
    if (moe_ws(w13, w2, t, topk, MoeCfg{c, c}).total > (int64_t)ws_bytes) continue;
    st = hum_moe_gemm_ex(w13, packed_w13, w2, packed_w2, t, topk, x_bf16, topk_ids, topk_weights, out_bf16,
                         workspace, ws_bytes, &c, stream);
    if (st == HUM_ERR_UNSUPPORTED) continue;
    if (st == HUM_OK && hipEventRecord(e0, s) != hipSuccess) st = set_error(HUM_ERR_HIP, "hipEventRecord failed");
    for (int i = 0; i < iters && st == HUM_OK; ++i)
      st = hum_moe_gemm_ex(w13, packed_w13, w2, packed_w2, t, topk, x_bf16, topk_ids, topk_weights, out_bf16,
                           workspace, ws_bytes, &c, stream);
    float ms = 0.0f;
    if (st == HUM_OK && (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                         hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
      st = set_error(HUM_ERR_HIP, "timing events failed");
    if (st != HUM_OK) {
      (void)hipEventDestroy(e0);
      (void)hipEventDestroy(e1);
      return st;
    }
    const float us = ms * 1000.0f / (float)iters;
    if (!found || us < best_us) {
      best_us = us;
      best = c;
      found = true;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (!found) return set_error(HUM_ERR_UNSUPPORTED, "no compiled configuration fits this shape and workspace");
  st = hum_moe_gemm_ex(w13, packed_w13, w2, packed_w2, t, topk, x_bf16, topk_ids, topk_weights, out_bf16, workspace,
                       ws_bytes, &best, stream);
  if (st != HUM_OK) return st;
  *best_out = best;
  if (best_us_out) *best_us_out = best_us;
  clear_error();
  return HUM_OK;
}

// ---- the grouped_masked layout ---------------------------------------------

// Validation shared by the masked entry points.
static hum_status check_masked(const hum_weight_desc* w13, const hum_weight_desc* w2, int64_t max_m,
                               int64_t expected_m) {
  if (max_m < 0 || max_m % 16) return set_error(HUM_ERR_INVALID_ARG, "max_m must be a non-negative multiple of 16");
  if (expected_m < 0) return set_error(HUM_ERR_INVALID_ARG, "expected_m < 0");
  if (!w13 || !w2) return set_error(HUM_ERR_INVALID_ARG, "NULL description");
  return check_moe(w13, w2, (int64_t)w13->num_experts * max_m, 1);
}

// Tile choice for the masked layout.  The grids must cover every expert
// buffer whole (E * max_m / block_m blocks times the N-tiles), however few
// rows are live, and a workgroup that finds its block dead still costs a
// dispatch: so the tile kernel with the largest block up to 64 rows that
// divides max_m, at every expected_m (measured on MI355X, 128 experts,
// max_m = 256, T = 16: the decode kernel's 16-row blocks made the layer
// several times slower than its live work).  expected_m is kept for the
// interface (the tile choice does not depend on it).
static MoeCfg select_masked(const hum_weight_desc* w13, int64_t max_m, int64_t expected_m) {
  (void)w13;
  (void)expected_m;
  const int wm = max_m % 64 == 0 ? 4 : (max_m % 32 == 0 ? 2 : 1);
  return MoeCfg{moe_tile_cfg(wm), moe_tile_cfg(wm)};
}

size_t hum_moe_masked_workspace_bytes(const hum_weight_desc* w13, const hum_weight_desc* w2, int64_t max_m,
                                      int64_t expected_m, const hum_tile_config* cfg) {
  clear_error();
  if (check_masked(w13, w2, max_m, expected_m) != HUM_OK) return 0;
  const MoeCfg mc = cfg ? MoeCfg{*cfg, *cfg} : select_masked(w13, max_m, expected_m);
  return (size_t)moe_ws(w13, w2, (int64_t)w13->num_experts * (max_m < 16 ? 16 : max_m), 1, mc, true).total;
}

hum_status hum_moe_gemm_masked(const hum_weight_desc* w13, const void* packed_w13, const hum_weight_desc* w2,
                               const void* packed_w2, int64_t max_m, int64_t expected_m, const void* x_bf16,
                               const int32_t* expert_num_tokens, void* out_bf16, void* workspace, size_t ws_bytes,
                               const hum_tile_config* cfg, void* stream) {
  clear_error();
  hum_status st = check_masked(w13, w2, max_m, expected_m);
  if (st != HUM_OK) return st;
  if (max_m == 0) return HUM_OK;
  if (!packed_w13 || !packed_w2 || !x_bf16 || !expert_num_tokens || !out_bf16)
    return set_error(HUM_ERR_INVALID_ARG, "NULL pointer");
  const MoeCfg mc = cfg ? MoeCfg{*cfg, *cfg} : select_masked(w13, max_m, expected_m);
  KernelKey kup, kdn;
  st = moe_keys(w13, mc, &kup, &kdn);
  if (st != HUM_OK) return st;
  const int32_t bm = (int32_t)tile_rows(mc.up);
  if (max_m % bm) return set_error(HUM_ERR_UNSUPPORTED, "the expert block (%d rows) must divide max_m", bm);
  const int64_t rows = (int64_t)w13->num_experts * max_m;
  const MoeWs w = moe_ws(w13, w2, rows, 1, mc, true);
  if (!workspace || ws_bytes < (size_t)w.total)
    return set_error(HUM_ERR_WORKSPACE, "workspace too small (%zu < %lld)", ws_bytes, (long long)w.total);
  log_cfg("moe masked up", mc.up, rows);
  log_cfg("moe masked down", mc.dn, rows);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  st = launch_masked_align(expert_num_tokens, w13->num_experts, max_m, bm, reinterpret_cast<int32_t*>(ws + w.sorted),
                           reinterpret_cast<int32_t*>(ws + w.bexp), stream);
  if (st != HUM_OK) return st;
  const MoeRows r{rows, 1, (int32_t)rows, (int32_t)(max_m < 16 ? max_m : 16), expert_num_tokens, max_m};
  return moe_gemms(w13, packed_w13, w2, packed_w2, mc, kup, kdn, w, ws, r, x_bf16, out_bf16, stream);
}

hum_status hum_moe_gemm(const hum_weight_desc* w13, const void* packed_w13, const hum_weight_desc* w2,
                        const void* packed_w2, int64_t t, int32_t topk, const void* x_bf16,
                        const int32_t* topk_ids, const float* topk_weights, void* out_bf16, void* workspace,
                        size_t ws_bytes, void* stream) {
  return hum_moe_gemm_ex(w13, packed_w13, w2, packed_w2, t, topk, x_bf16, topk_ids, topk_weights, out_bf16,
                         workspace, ws_bytes, nullptr, stream);
}

}  // extern "C"
