// C ABI entry points: description checks, packed layout, the tile / split-K
// selector, workspace carving and dispatch.  Host code only.
//
// The selector follows the idea of "Device-parameter tuning" in "Announcing
// Humming: Fast, Flexible Kernels for Quantized Inference": the shape, the
// format and the device's resources (here: 256 CUs, 160 KB LDS, wave64)
// choose a tile and split per M range, at run time, with no compilation.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
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
      if (d->has_zero_point && d->weight_dtype != HUM_UINT4) return set_error(HUM_ERR_UNSUPPORTED, "zero points need UINT4 codes");
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
  if (d->weight_dtype == HUM_INT4 || d->weight_dtype == HUM_UINT4) return F_INT;
  if (d->weight_dtype == HUM_INT8) return F_INT8_BF16;
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
  L->code_bytes = (f == F_FP8 || f == F_FP8_BLOCK || fmt_w8_bf16(f)) ? 32 : 16;
  L->codes_per_expert = L->nt * L->kb * 64 * L->code_bytes;
  if (f == F_INT) {
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
  return c.kind == HUM_KERNEL_TILE ? (c.stages == 0 ? 2 : c.stages) : 0;
}

static KernelKey dense_key(const hum_weight_desc* d, const hum_tile_config& c) {
  return KernelKey{fmt_of(d), c.kind, c.wave_m, c.wave_n, c.waves_n, c.waves_k, A_DIRECT, EPI_BF16, key_stages(c)};
}

static bool cfg_sane(const hum_tile_config& c) {
  if (c.split_k < 1 || c.split_k > 64 || c.wave_m < 1 || c.wave_n < 1) return false;
  if (c.kind == HUM_KERNEL_STREAM) return c.wave_m == 1 && c.waves_n == 1 && c.waves_k >= 1 && c.waves_k <= 15;
  if (c.kind == HUM_KERNEL_TILE) return c.waves_n == 4 && c.waves_k == 1 && (c.stages == 0 || c.stages == 2 || c.stages == 3);
  return false;
}

static int64_t tile_rows(const hum_tile_config& c) { return 16 * (int64_t)c.wave_m; }

// Columns (16-wide sub-tiles) one workgroup covers.
static int64_t tile_subtiles(const hum_tile_config& c) {
  return (int64_t)c.wave_n * (c.kind == HUM_KERNEL_TILE ? 4 : 1);
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

static hum_tile_config select_dense(const hum_weight_desc* d, int64_t m) {
  hum_tile_config c{};
  const int64_t nt = cdiv(d->n, kNSub);
  const int64_t kb = d->k / kKBlk;
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
    const int64_t w_bytes16 = (fmt_of(d) == F_FP8 || fmt_w8_bf16(fmt_of(d))) ? 16 : 8;      // per k of a 16-column sub-tile
    const int64_t need = cdiv(a_bytes, w_bytes16);
    c.wave_n = need <= 1 ? 1 : (need <= 2 ? 2 : 4);
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
  } else {
    c.kind = HUM_KERNEL_TILE;
    c.waves_n = 4;
    c.waves_k = 1;
    // Measured on MI355X (dense N = K = 8192 and N = 7168, K = 2048): small
    // tiles with split-K while the tile count is low; 64 x 256 tiles for
    // bf16 activations from M = 512 (fewer LDS activation reads per MFMA);
    // 128 x 128 for FP8 activations.  W4A4 (no decode kernel) takes the
    // small tiles from M = 1.
    const bool bf16_act = fmt_bf16_act(fmt_of(d));
    int64_t target = 3 * kCUs;
    if (m <= 256) {
      c.wave_m = 2;
      c.wave_n = 2;
      c.stages = 3;  // small tiles: room in LDS for a deeper pipeline
      if (bf16_act) target = 8 * kCUs;
    } else if (bf16_act) {
      c.wave_m = 4;
      c.wave_n = m >= 512 ? 4 : 2;
    } else {
      c.wave_m = 8;
      c.wave_n = 2;
    }
    const int64_t wgs = cdiv(m, tile_rows(c)) * cdiv(nt, tile_subtiles(c));
    // 8-bit weights with bf16 activations: split K only while every split
    // keeps at least 16 K-blocks (so none at K = 2048, where one pass
    // measured 1.6-2.4x faster than split-K for M = 64..256 on MI355X)
    c.split_k = pick_split(wgs, 4, kb, 1, fmt_w8_bf16(fmt_of(d)) ? 16 : 4, target);
    if (fmt_of(d) == F_FP8_BLOCK) {
      // block-scaled FP8 (no decode kernel): small tiles with three stages
      // to M = 256, then the FP8 128 x 128 tiles
      if (m <= 256) {
        c.wave_m = 2;
        c.wave_n = 2;
        c.stages = 3;
      }
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

// Measured on MI355X (E = 128, top-8, H = 4096, I = 1024) over the mean
// rows per expert: the decode kernel only while most experts see at most a
// row or two (it reads each weight once, but its bf16 path is VALU heavy);
// 16-row tiles up to ~100 rows, larger tiles beyond.
static MoeCfg select_moe(const hum_weight_desc* w13, int64_t t, int32_t topk) {
  const double rows = (double)t * topk / w13->num_experts;
  if (fmt_of(w13) == F_MXFP4_MXFP4) {
    // W4A4: tile kernels only (no decode-kernel path)
    const int wm = rows <= 16 ? 1 : (rows <= 256 ? 2 : 4);
    return {moe_tile_cfg(wm), moe_tile_cfg(wm)};
  }
  if (fmt_of(w13) != F_MXFP4_MXFP8) {
    if (rows < 0.5) return {moe_stream_cfg(), moe_stream_cfg()};
    const int wm = rows <= 96 ? 1 : (rows <= 192 ? 2 : 4);
    return {moe_tile_cfg(wm), moe_tile_cfg(wm)};
  }
  if (rows <= 2) return {moe_stream_cfg(), moe_stream_cfg()};
  if (rows <= 16) return {moe_stream_cfg(), moe_tile_cfg(1)};
  const int wm = rows <= 256 ? 2 : 4;
  return {moe_tile_cfg(wm), moe_tile_cfg(wm)};
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
  int64_t off = 0;
  w.partials = off;
  if (c.split_k > 1) off = align256(off + (int64_t)c.split_k * m * nt * 16 * 4);
  w.aq = off;
  if (quant_a) {
    off = align256(off + (d->act_fmt == HUM_ACT_MXFP4 ? m * (d->k / 2) : m * d->k));
    w.as = off;
    off = align256(off + (d->act_fmt == HUM_ACT_MXFP8 || d->act_fmt == HUM_ACT_MXFP4
                              ? m * (d->k / 32)
                              : (d->act_fmt == HUM_ACT_FP8_GROUP ? m * (d->k / 128) * 4 : m * 4)));
  }
  w.rowsum = off;
  if (fmt_of(d) == F_INT && c.kind == HUM_KERNEL_TILE) off = align256(off + cdiv(m, 16) * cdiv(d->k / kKBlk, 32) * 2048);
  w.total = off;
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
  c.split_k = 1;
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
  p.int_offset = (d->weight_dtype == HUM_INT4) ? 136 : 128;
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
  hum_tile_config c = cfg ? *cfg : select_dense(desc, m);
  if (!cfg_sane(c) || !gemm_instance_exists(dense_key(desc, c)))
    return set_error(HUM_ERR_UNSUPPORTED, "tile config not available");
  if (c.kind == HUM_KERNEL_STREAM && m > 16) return set_error(HUM_ERR_UNSUPPORTED, "the stream kernel takes m <= 16");
  const bool quant_a = desc->act_fmt != HUM_ACT_BF16 && a_scales == nullptr;
  const DenseWs w = dense_ws(desc, m, c, quant_a);
  if (w.total > 0 && (!workspace || ws_bytes < (size_t)w.total))
    return set_error(HUM_ERR_WORKSPACE, "workspace too small (%zu < %lld)", ws_bytes, (long long)w.total);
  log_cfg("linear", c, m);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const void* a_use = a;
  const void* as_use = a_scales;
  if (quant_a) {
    st = hum_quant_act(desc->act_fmt, m, desc->k, a, desc->k, ws + w.aq, ws + w.as, stream);
    if (st != HUM_OK) return st;
    a_use = ws + w.aq;
    as_use = ws + w.as;
  }
  GemmParams p{};
  fill_weight_params(p, desc, L, packed);
  if (fmt_of(desc) == F_INT && c.kind == HUM_KERNEL_TILE) {
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
  p.stream_rows = (int)(m < 16 ? m : 16);
  p.a_bytes = fmt_of(desc) == F_MXFP4_MXFP4 ? m * (desc->k / 2)
                                            : m * desc->k * (fmt_bf16_act(fmt_of(desc)) ? 2 : 1);
  p.a_scale_bytes = (desc->act_fmt == HUM_ACT_MXFP8 || desc->act_fmt == HUM_ACT_MXFP4) ? m * (desc->k / 32)
                    : (desc->act_fmt == HUM_ACT_FP8_GROUP ? m * (desc->k / 128) * 4 : 0);
  return launch_gemm(dense_key(desc, c), p, m_tiles, (int)tile_rows(c), stream);
}

hum_status hum_linear(const hum_weight_desc* desc, const void* packed, int64_t m, const void* a, const void* a_scales,
                      const void* bias, void* out, void* workspace, size_t ws_bytes, void* stream) {
  return hum_linear_ex(desc, packed, m, a, a_scales, bias, out, workspace, ws_bytes, nullptr, stream);
}

// ---------------------------------------------------------------------------
// On-device autotune: every compiled dense configuration, timed on the
// caller's own buffers.

static void dense_candidates(const hum_weight_desc* d, int64_t m, uint32_t flags, std::vector<hum_tile_config>& out) {
  const int64_t kb = d->k / kKBlk;
  const bool inv = (flags & HUM_SELECT_BATCH_INVARIANT) != 0;
  for (int split = 1; split <= 16; split *= 2) {
    if (inv && split > 1) break;
    for (int kind = HUM_KERNEL_TILE; kind <= HUM_KERNEL_STREAM; ++kind) {
      if (kind == HUM_KERNEL_STREAM && (inv || m > 16)) continue;
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
              c.split_k = split;
              c.stages = st;
              c.block_m = (int32_t)tile_rows(c);
              // every split must own at least one K-block
              if (split > 1 && (int64_t)kb_per_split(kb, c) * (split - 1) >= kb) continue;
              if (cfg_sane(c) && gemm_instance_exists(dense_key(d, c))) out.push_back(c);
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

struct MoeWs {
  int64_t partials = 0, sorted = 0, offsets = 0, counts = 0, bexp = 0;
  int64_t xq = 0, xs = 0, inter = 0, inter_s = 0, y = 0, total = 0;
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
  w.cap = masked ? t : t * topk + E * (bm - 1);
  w.nblocks = cdiv(w.cap, bm);
  const bool mx = w13->act_fmt == HUM_ACT_MXFP8 || w13->act_fmt == HUM_ACT_MXFP4;
  const bool mx4 = w13->act_fmt == HUM_ACT_MXFP4;  // E2M1 codes, two per byte
  const int64_t pcols = (2 * inter > cdiv(h, kNSub) * kNSub) ? 2 * inter : cdiv(h, kNSub) * kNSub;
  int64_t off = 0;
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
  w.xq = off;
  if (mx) {
    off = align256(off + (mx4 ? t * (h / 2) : t * h));
    w.xs = off;
    off = align256(off + t * (h / 32));
  }
  w.inter = off;
  off = align256(off + (mx4 ? w.cap * (inter / 2) : w.cap * inter * (mx ? 1 : 2)));
  w.inter_s = off;
  if (mx) off = align256(off + w.cap * (inter / 32));
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
  if (w13->weight_dtype != HUM_E2M1 || w2->weight_dtype != HUM_E2M1 || w13->scale_dtype != HUM_E8M0 ||
      w2->scale_dtype != HUM_E8M0)
    return set_error(HUM_ERR_UNSUPPORTED, "the MoE path runs MXFP4 (E2M1 + E8M0) expert weights");
  if (w13->act_fmt != w2->act_fmt) return set_error(HUM_ERR_INVALID_ARG, "w13 and w2 activation formats differ");
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
  if (flags & ~(uint32_t)HUM_SELECT_BATCH_INVARIANT) return set_error(HUM_ERR_INVALID_ARG, "unknown selection flags 0x%x", flags);
  hum_tile_config c = select_moe(w13, t < 1 ? 1 : t, topk).dn;
  // the grouped tile kernel sums each slot's row in a fixed order (no split-K);
  // the decode kernel splits K inside the workgroup
  if ((flags & HUM_SELECT_BATCH_INVARIANT) && c.kind != HUM_KERNEL_TILE) c = moe_tile_cfg(1);
  *cfg_out = c;
  return HUM_OK;
}

size_t hum_moe_workspace_bytes_ex(const hum_weight_desc* w13, const hum_weight_desc* w2, int64_t t, int32_t topk,
                                  const hum_tile_config* cfg) {
  clear_error();
  if (check_moe(w13, w2, t, topk) != HUM_OK) return 0;
  const MoeCfg mc = cfg ? MoeCfg{*cfg, *cfg} : select_moe(w13, t, topk);
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

hum_status hum_moe_reduce(const void* y_bf16, const float* topk_weights, int64_t t, int32_t topk, int64_t h,
                          void* out_bf16, void* stream) {
  clear_error();
  if (t < 0 || topk < 1 || h < 8 || h % 8) return set_error(HUM_ERR_INVALID_ARG, "bad sizes (h must be a multiple of 8)");
  if (t > 0 && (!y_bf16 || !topk_weights || !out_bf16)) return set_error(HUM_ERR_INVALID_ARG, "NULL pointer");
  return launch_moe_reduce(y_bf16, topk_weights, t, topk, h, out_bf16, stream);
}

// Kernel keys of a layer's two GEMMs; HUM_OK when both are compiled.
static hum_status moe_keys(const hum_weight_desc* w13, const MoeCfg& mc, KernelKey* kup, KernelKey* kdn) {
  const hum_tile_config& cu = mc.up;
  const hum_tile_config& cd = mc.dn;
  if (!cfg_sane(cu) || !cfg_sane(cd) || tile_rows(cu) != tile_rows(cd))
    return set_error(HUM_ERR_UNSUPPORTED, "tile config not available");
  const int f = fmt_of(w13);
  const int epi_up =
      (f == F_MXFP4_MXFP8) ? EPI_SWIGLU_MXFP8 : (f == F_MXFP4_MXFP4 ? EPI_SWIGLU_MXFP4 : EPI_SWIGLU_BF16);
  *kup = KernelKey{f, cu.kind, cu.wave_m, cu.wave_n, cu.waves_n, cu.waves_k, A_GATHER, epi_up, key_stages(cu)};
  *kdn = KernelKey{f, cd.kind, cd.wave_m, cd.wave_n, cd.waves_n, cd.waves_k, A_DIRECT, EPI_SCATTER, key_stages(cd)};
  if (!gemm_instance_exists(*kup) || !gemm_instance_exists(*kdn)) return set_error(HUM_ERR_UNSUPPORTED, "tile config not available");
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
};

// gate_up (+ SwiGLU, + requantization) into the workspace, then down with
// its rows scattered to y[slot] (row stride h), over the expert blocks that
// ws.sorted / ws.bexp describe.
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
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + w.sorted);
  int32_t* bexp = reinterpret_cast<int32_t*>(ws + w.bexp);
  const int f = fmt_of(w13);
  const bool mx4 = f == F_MXFP4_MXFP4;
  const bool mx = f == F_MXFP4_MXFP8 || mx4;
  const void* x_use = x_bf16;
  hum_status st = HUM_OK;
  if (mx) {
    st = mx4 ? launch_quant_mxfp4(t, h, x_bf16, h, ws + w.xq, ws + w.xs, stream, r.counts, r.max_m)
             : launch_quant_mxfp8(t, h, x_bf16, h, ws + w.xq, ws + w.xs, stream, r.counts, r.max_m);
    if (st != HUM_OK) return st;
    x_use = ws + w.xq;
  }
  // gate_up (+ SwiGLU)
  GemmParams p{};
  fill_weight_params(p, w13, L13, packed_w13);
  p.n = inter;
  p.swiglu_nt_off = (int)(inter / kNSub);
  p.a = x_use;
  p.lda = h;
  p.a_scale = mx ? ws + w.xs : nullptr;
  p.a_scale_ld = h / 32;
  p.m = w.cap;
  p.sorted = sorted;
  p.block_expert = bexp;
  p.topk = r.topk;
  p.sentinel = r.sentinel;
  p.out = ws + w.inter;
  p.ldo = inter;
  p.out_scale = mx ? ws + w.inter_s : nullptr;
  p.bias = nullptr;
  p.n_tiles = (int)cdiv(cdiv(inter, kNSub), tile_subtiles(cu) / 2);
  p.split_k = cu.split_k;
  p.kb_per_split = kb_per_split(L13.kb, cu);
  p.partials = reinterpret_cast<float*>(ws + w.partials);
  p.stream_rows = r.stream_rows;
  p.a_bytes = mx4 ? t * (h / 2) : t * h * (mx ? 1 : 2);
  p.a_scale_bytes = mx ? t * (h / 32) : 0;
  st = launch_gemm(kup, p, w.nblocks, bm, stream);
  if (st != HUM_OK) return st;
  // down (rows scattered back to flat slots)
  GemmParams q{};
  fill_weight_params(q, w2, L2, packed_w2);
  q.a = ws + w.inter;
  q.lda = inter;
  q.a_scale = mx ? ws + w.inter_s : nullptr;
  q.a_scale_ld = inter / 32;
  q.m = w.cap;
  q.sorted = sorted;
  q.block_expert = bexp;
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
  q.a_bytes = mx4 ? w.cap * (inter / 2) : w.cap * inter * (mx ? 1 : 2);
  q.a_scale_bytes = mx ? w.cap * (inter / 32) : 0;
  return launch_gemm(kdn, q, w.nblocks, bm, stream);
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
  const MoeCfg mc = cfg ? MoeCfg{*cfg, *cfg} : select_moe(w13, t, topk);
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
  st = launch_align(topk_ids, t, topk, (int32_t)E, (int32_t)tile_rows(mc.up), reinterpret_cast<int32_t*>(ws + w.sorted),
                    reinterpret_cast<int32_t*>(ws + w.offsets), reinterpret_cast<int32_t*>(ws + w.counts),
                    reinterpret_cast<int32_t*>(ws + w.bexp), w.nblocks, stream);
  if (st != HUM_OK) return st;
  const int64_t slots = t * topk;
  const MoeRows rows{t, topk, (int32_t)slots, (int32_t)(slots < 16 ? slots : 16), nullptr, 0};
  st = moe_gemms(w13, packed_w13, w2, packed_w2, mc, kup, kdn, w, ws, rows, x_bf16, ws + w.y, stream);
  if (st != HUM_OK) return st;
  return launch_moe_reduce(ws + w.y, topk_weights, t, topk, h, out_bf16, stream);
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
