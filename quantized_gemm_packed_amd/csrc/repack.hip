// Weight preparation: canonical ("standard format") tensors -> packed
// kernel layout, and the exact dequantization of a packed buffer (test
// export).  The preparation step -- validate, pad, repack into the layout the
// kernel needs -- is the one described in "Announcing Humming: Fast, Flexible
// Kernels for Quantized Inference", section "Per-workload tuning and JIT
// compilation".  The packed layout itself is documented in hum_internal.h.
#include "dev_common.h"
#include "hum_internal.h"

namespace hum {

struct RepackArgs {
  const uint8_t* codes;
  const uint8_t* scales;
  const uint8_t* zeros;
  const float* gscale;
  uint8_t* packed;
  int64_t n, k;
  int64_t nt, kb, ng, kb4;
  int64_t codes_off, scales_off, zeros_off, co_off, gscale_off;
  int64_t codes_pe, scales_pe, zeros_pe, co_pe;
  int64_t kbc, kb_per_group;
  int64_t src_ng;      // scale columns per canonical row (K/G or 1)
  int64_t src_n;       // canonical scale rows per expert (N or 1)
  int num_experts;
  int wdt;             // hum_dtype of the weights
  int scale_elem;      // bytes per scale element (1, 2 or 4)
  int has_zero;
  int has_gscale;
  int bf16_order;      // 8-bit codes for the bf16 MFMA (bf16 activations)
};

// 32 canonical 4-bit codes of (row n, k0 .. k0+31) as 4 dwords in the
// packed order of the format.
__device__ __forceinline__ u32x4_t pack_lane_4bit(const RepackArgs& a, int64_t e, int64_t n, int64_t k0) {
  u32x4_t r;
  if (n >= a.n) {
    // padding rows decode to zero: INT4 stores v + 8
    uint32_t pad = (a.wdt == HUM_INT4) ? 0x88888888u : 0u;
    r[0] = r[1] = r[2] = r[3] = pad;
    return r;
  }
  const uint8_t* src = a.codes + ((e * a.n + n) * a.k + k0) / 2;
  u32x4_t raw = *reinterpret_cast<const u32x4_t*>(src);
  if (a.wdt == HUM_E2M1) return raw;  // canonical nibble order is the MFMA order
  const uint32_t flip = (a.wdt == HUM_INT4) ? 0x88888888u : 0u;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint32_t w = raw[s] ^ flip;  // nibbles k = 8s + 0..7, even k low
    uint32_t o = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t u = (w >> (4 * j)) & 0xFu;
      o |= u << ((j & 1) * 16 + (j >> 1) * 4);
    }
    r[s] = o;
  }
  return r;
}

// 32 canonical b-bit codes (b = 1, 2, 3) of (row n, k0 .. k0+31) in the
// packed bit planes of the integer path: the 2-bit plane (b = 2, 3) in dwords
// 0, 1 -- element j of 8-k step s at dword s / 2, bit (j & 1) * 16 +
// 2 * (4 * (s & 1) + j / 2) -- and the 1-bit plane (bit 2 of a 3-bit code,
// the code itself for b = 1) in the next dword, element j of step s at bit
// (j & 1) * 16 + 4 * s + j / 2.  Signed codes are stored offset by 2^(b-1);
// padding rows hold the codes that decode to zero.
__device__ __forceinline__ void pack_lane_bits(const RepackArgs& a, int bits, bool sgn, int64_t e, int64_t n,
                                               int64_t k0, uint32_t (&out)[3]) {
  const uint32_t flip = sgn ? (1u << (bits - 1)) : 0u;
  uint32_t src[3] = {0, 0, 0};
  if (n < a.n) {
    // the row's 32 codes: 4b bytes from bit b * k0 of the row (dword aligned:
    // K is a multiple of 128)
    const uint32_t* w = reinterpret_cast<const uint32_t*>(a.codes + ((e * a.n + n) * a.k + k0) * bits / 8);
    for (int i = 0; i < bits; ++i) src[i] = w[i];
  }
  out[0] = out[1] = out[2] = 0;
  for (int s = 0; s < 4; ++s)
    for (int j = 0; j < 8; ++j) {
      const int bit = bits * (8 * s + j);
      const uint64_t win = (uint64_t)src[bit / 32] | ((bit / 32 + 1 < bits) ? (uint64_t)src[bit / 32 + 1] << 32 : 0);
      uint32_t u = (uint32_t)(win >> (bit % 32)) & ((1u << bits) - 1);
      u = (n < a.n) ? (u ^ flip) : flip;
      if (bits >= 2) out[s >> 1] |= (u & 3u) << ((j & 1) * 16 + 2 * (4 * (s & 1) + (j >> 1)));
      if (bits != 2) out[bits == 3 ? 2 : 0] |= ((bits == 3 ? (u >> 2) : u) & 1u) << ((j & 1) * 16 + 4 * s + (j >> 1));
    }
}

__global__ void repack_codes_kernel(RepackArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.num_experts * a.nt * a.kb * 64;
  if (tid >= total) return;
  const int lane = (int)(tid & 63);
  int64_t rest = tid >> 6;
  const int64_t kb = rest % a.kb;
  rest /= a.kb;
  const int64_t nt = rest % a.nt;
  const int64_t e = rest / a.nt;
  const int c = lane & 15, lg = lane >> 4;
  const int64_t n = nt * kNSub + c;
  uint8_t* dst = a.packed + a.codes_off + e * a.codes_pe;
  if (a.wdt == HUM_E4M3 || a.wdt == HUM_INT8) {
    // the 16x16x128 FP8 MFMA takes k = 16 lg + [0, 16) and 64 + 16 lg +
    // [0, 16) per lane; the bf16 MFMA's four k-steps take k = 32 lg + 8 s +
    // [0, 8), i.e. 32 contiguous codes
    u32x4_t lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
    if (n < a.n) {
      const uint8_t* src = a.codes + (e * a.n + n) * a.k + kb * kKBlk;
      lo = *reinterpret_cast<const u32x4_t*>(src + (a.bf16_order ? 32 * lg : 16 * lg));
      hi = *reinterpret_cast<const u32x4_t*>(src + (a.bf16_order ? 32 * lg + 16 : 64 + 16 * lg));
    }
    u32x4_t* d = reinterpret_cast<u32x4_t*>(dst + ((nt * a.kb + kb) * 64 + lane) * 32);
    d[0] = lo;
    d[1] = hi;
  } else if (a.wdt == HUM_E2M3 || a.wdt == HUM_E3M2) {
    // FP6: the canonical 6-bit stream of the lane's 32 codes, as is (24
    // dword-aligned bytes: K is a multiple of 128)
    uint32_t v[6] = {0, 0, 0, 0, 0, 0};
    if (n < a.n) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(a.codes + ((e * a.n + n) * a.k + kb * kKBlk + 32 * lg) * 6 / 8);
      for (int i = 0; i < 6; ++i) v[i] = w[i];
    }
    uint32_t* d = reinterpret_cast<uint32_t*>(dst + ((nt * a.kb + kb) * 64 + lane) * 24);
    for (int i = 0; i < 6; ++i) d[i] = v[i];
  } else if (dtype_int_bits(a.wdt) != 0 && dtype_int_bits(a.wdt) < 4) {
    const int bits = dtype_int_bits(a.wdt);
    uint32_t v[3];
    pack_lane_bits(a, bits, dtype_int_signed(a.wdt), e, n, kb * kKBlk + 32 * lg, v);
    uint32_t* d = reinterpret_cast<uint32_t*>(dst + ((nt * a.kb + kb) * 64 + lane) * 4 * bits);
    for (int i = 0; i < bits; ++i) d[i] = v[i];
  } else {
    u32x4_t v = pack_lane_4bit(a, e, n, kb * kKBlk + 32 * lg);
    *reinterpret_cast<u32x4_t*>(dst + ((nt * a.kb + kb) * 64 + lane) * 16) = v;
  }
}

// INT meta: one thread per (e, nt, g): 16 scales (+ 16 zero nibbles).
__global__ void repack_int_meta_kernel(RepackArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.num_experts * a.nt * a.ng;
  if (tid >= total) return;
  const int64_t g = tid % a.ng;
  const int64_t nt = (tid / a.ng) % a.nt;
  const int64_t e = tid / (a.ng * a.nt);
  uint8_t* sdst = a.packed + a.scales_off + e * a.scales_pe + (nt * a.ng + g) * 16 * a.scale_elem;
  uint64_t zp = 0;
  for (int c = 0; c < 16; ++c) {
    const int64_t n = nt * kNSub + c;
    const int64_t sr = (a.src_n == 1) ? 0 : n;
    const int64_t sg = (a.src_ng == 1) ? 0 : g;
    const bool valid = n < a.n;
    const int64_t sidx = (e * a.src_n + sr) * a.src_ng + sg;
    if (a.scale_elem == 2) {
      uint16_t v = valid ? reinterpret_cast<const uint16_t*>(a.scales)[sidx] : 0;
      reinterpret_cast<uint16_t*>(sdst)[c] = v;
    } else {
      float v = valid ? reinterpret_cast<const float*>(a.scales)[sidx] : 0.0f;
      reinterpret_cast<float*>(sdst)[c] = v;
    }
    if (a.has_zero && valid) zp |= (uint64_t)(a.zeros[sidx] & 0xF) << (4 * c);
  }
  if (a.zeros_pe) {
    *reinterpret_cast<uint64_t*>(a.packed + a.zeros_off + e * a.zeros_pe + (nt * a.ng + g) * 8) = zp;
  }
}

// INT offset terms: one thread per (e, nt, kbc, lane) writes the 8 K-blocks
// 32 kbc + 8 lg + j of column c as -s * (offset + z), split into a bf16
// high part and the bf16 of the remainder.  s * (offset + z) is exact in
// f32 for bf16 scales (at most 8 + 8 significant bits).
__global__ void repack_int_co_kernel(RepackArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.num_experts * a.nt * a.kbc * 64;
  if (tid >= total) return;
  const int lane = (int)(tid & 63);
  int64_t rest = tid >> 6;
  const int64_t cc = rest % a.kbc;
  rest /= a.kbc;
  const int64_t nt = rest % a.nt;
  const int64_t e = rest / a.nt;
  const int c = lane & 15, lg = lane >> 4;
  const int64_t n = nt * kNSub + c;
  // what the bf16 (128 + u) codes carry beyond the value: 128 + 2^(b-1) for
  // signed b-bit codes (stored offset by 2^(b-1)), 128 for unsigned ones
  const float offset = dtype_int_signed(a.wdt) ? (float)(128 + (1 << (dtype_int_bits(a.wdt) - 1))) : 128.0f;
  u32x4_t hi, lo;
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    float v[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int64_t kb = cc * 32 + 8 * lg + j + q;
      v[q] = 0.0f;
      if (n < a.n && kb < a.kb) {
        const int64_t g = kb / a.kb_per_group;
        const int64_t sr = (a.src_n == 1) ? 0 : n;
        const int64_t sg = (a.src_ng == 1) ? 0 : g;
        const int64_t sidx = (e * a.src_n + sr) * a.src_ng + sg;
        const float sc = (a.scale_elem == 2) ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(a.scales)[sidx])
                                             : reinterpret_cast<const float*>(a.scales)[sidx];
        const float z = a.has_zero ? (float)(a.zeros[sidx] & 0xF) : 0.0f;
        v[q] = -(sc * (offset + z));
      }
    }
    const uint32_t h0 = f32_to_bf16_bits(v[0]), h1 = f32_to_bf16_bits(v[1]);
    const uint32_t l0 = f32_to_bf16_bits(v[0] - bf16_bits_to_f32(h0));
    const uint32_t l1 = f32_to_bf16_bits(v[1] - bf16_bits_to_f32(h1));
    hi[j / 2] = h0 | (h1 << 16);
    lo[j / 2] = l0 | (l1 << 16);
  }
  uint8_t* base = a.packed + a.co_off + e * a.co_pe;
  const int64_t idx = ((nt * a.kbc + cc) * 64 + lane) * 16;
  *reinterpret_cast<u32x4_t*>(base + idx) = hi;
  *reinterpret_cast<u32x4_t*>(base + a.nt * a.kbc * 1024 + idx) = lo;
}

// MX meta: one thread per (e, nt, kb4, lane): E8M0 codes of 4 K-blocks.
__global__ void repack_mx_meta_kernel(RepackArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.num_experts * a.nt * a.kb4 * 64;
  if (tid >= total) return;
  const int lane = (int)(tid & 63);
  int64_t rest = tid >> 6;
  const int64_t kb4 = rest % a.kb4;
  rest /= a.kb4;
  const int64_t nt = rest % a.nt;
  const int64_t e = rest / a.nt;
  const int c = lane & 15, lg = lane >> 4;
  const int64_t n = nt * kNSub + c;
  uint32_t word = 0;
  for (int i = 0; i < 4; ++i) {
    const int64_t kb = kb4 * 4 + i;
    uint32_t code = 127;
    if (n < a.n && kb < a.kb) code = a.scales[(e * a.n + n) * (a.k / 32) + kb * 4 + lg];
    word |= code << (8 * i);
  }
  *reinterpret_cast<uint32_t*>(a.packed + a.scales_off + e * a.scales_pe + ((nt * a.kb4 + kb4) * 64 + lane) * 4) = word;
}

// NVFP4 meta: one dword per (e, nt, K-block pair, lane), bytes 2 h + q =
// the E4M3 scale of group 8 kb + 2 lg + q for K-block kb = 2 kb2 + h (the
// lane's 32 codes of a K-block span groups 2 lg and 2 lg + 1).  Codes of
// columns past N are zero, so their scale is too.
__global__ void repack_nv_meta_kernel(RepackArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.num_experts * a.nt * a.kb4 * 64;
  if (tid >= total) return;
  const int lane = (int)(tid & 63);
  int64_t rest = tid >> 6;
  const int64_t kb2 = rest % a.kb4;
  rest /= a.kb4;
  const int64_t nt = rest % a.nt;
  const int64_t e = rest / a.nt;
  const int c = lane & 15, lg = lane >> 4;
  const int64_t n = nt * kNSub + c;
  uint32_t word = 0;
  for (int h = 0; h < 2; ++h) {
    const int64_t kb = 2 * kb2 + h;
    if (kb >= a.kb || n >= a.n) continue;
    for (int q = 0; q < 2; ++q) {
      const int64_t g = kb * 8 + 2 * lg + q;
      word |= (uint32_t)a.scales[(e * a.src_n + n) * a.src_ng + g] << (8 * (2 * h + q));
    }
  }
  *reinterpret_cast<uint32_t*>(a.packed + a.scales_off + e * a.scales_pe + ((nt * a.kb4 + kb2) * 64 + lane) * 4) = word;
}

// FP8 per-channel meta: f32 [NT*16] per expert.
__global__ void repack_fp8_meta_kernel(RepackArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = a.nt * kNSub;
  if (tid >= (int64_t)a.num_experts * per) return;
  const int64_t n = tid % per;
  const int64_t e = tid / per;
  float v = 1.0f;
  if (n < a.n) {
    const int64_t sr = (a.src_n == 1) ? 0 : n;
    v = reinterpret_cast<const float*>(a.scales)[e * a.src_n + sr];
  }
  reinterpret_cast<float*>(a.packed + a.scales_off + e * a.scales_pe)[n] = v;
}

// Block-scaled FP8 meta: one f32 per (e, 16-column sub-tile, K-block), the
// scale of the 128 x 128 block the sub-tile's rows and the K-block lie in.
__global__ void repack_fp8_block_meta_kernel(RepackArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = a.nt * a.kb;
  if (tid >= (int64_t)a.num_experts * per) return;
  const int64_t kb = tid % a.kb;
  const int64_t nt = (tid / a.kb) % a.nt;
  const int64_t e = tid / per;
  const int64_t n = nt * kNSub;
  float v = 1.0f;
  if (n < a.n) v = reinterpret_cast<const float*>(a.scales)[(e * a.src_n + n / 128) * a.src_ng + kb];
  reinterpret_cast<float*>(a.packed + a.scales_off + e * a.scales_pe)[nt * a.kb + kb] = v;
}

__global__ void repack_gscale_kernel(RepackArgs a) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= a.num_experts) return;
  reinterpret_cast<float*>(a.packed + a.gscale_off)[e] = a.has_gscale ? a.gscale[e] : 1.0f;
}

static inline unsigned grid_for(int64_t total, int block) {
  return (unsigned)((total + block - 1) / block);
}

hum_status launch_repack(const hum_weight_desc* d, const Layout& L, const void* codes,
                         const void* scales, const void* zeros, const float* gscale,
                         void* packed, void* stream) {
  RepackArgs a;
  a.codes = static_cast<const uint8_t*>(codes);
  a.scales = static_cast<const uint8_t*>(scales);
  a.zeros = static_cast<const uint8_t*>(zeros);
  a.gscale = gscale;
  a.packed = static_cast<uint8_t*>(packed);
  a.n = d->n;
  a.k = d->k;
  a.nt = L.nt;
  a.kb = L.kb;
  a.ng = L.ng;
  a.kb4 = L.kb4;
  a.codes_off = L.codes_off;
  a.scales_off = L.scales_off;
  a.zeros_off = L.zeros_off;
  a.co_off = L.co_off;
  a.gscale_off = L.gscale_off;
  a.codes_pe = L.codes_per_expert;
  a.scales_pe = L.scales_per_expert;
  a.zeros_pe = L.zeros_per_expert;
  a.co_pe = L.co_per_expert;
  a.kbc = L.kbc;
  a.kb_per_group = L.kb_per_group;
  a.src_n = (d->scale_gran == HUM_SCALE_TENSOR) ? 1 : (d->scale_gran == HUM_SCALE_BLOCK ? (d->n + 127) / 128 : d->n);
  a.src_ng = (d->scale_gran == HUM_SCALE_GROUP || d->scale_gran == HUM_SCALE_BLOCK) ? d->k / d->group_size : 1;
  a.num_experts = d->num_experts;
  a.wdt = d->weight_dtype;
  a.scale_elem = d->scale_dtype == HUM_BF16 ? 2 : (d->scale_dtype == HUM_F32 ? 4 : 1);
  a.has_zero = d->has_zero_point;
  a.has_gscale = d->has_global_scale;
  a.bf16_order = fmt_w8_bf16(fmt_of(d));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int B = 256;
  const int64_t ncode = (int64_t)d->num_experts * L.nt * L.kb * 64;
  repack_codes_kernel<<<grid_for(ncode, B), B, 0, s>>>(a);
  const int f = fmt_of(d);
  if (fmt_int(f)) {
    repack_int_meta_kernel<<<grid_for((int64_t)d->num_experts * L.nt * L.ng, B), B, 0, s>>>(a);
    repack_int_co_kernel<<<grid_for((int64_t)d->num_experts * L.nt * L.kbc * 64, B), B, 0, s>>>(a);
  } else if (f == F_NVFP4_BF16) {
    repack_nv_meta_kernel<<<grid_for((int64_t)d->num_experts * L.nt * L.kb4 * 64, B), B, 0, s>>>(a);
  } else if (f == F_MXFP4_BF16 || f == F_MXFP4_MXFP8 || f == F_MXFP4_MXFP4 || f == F_MXINT4_BF16 || fmt_fp6(f)) {
    repack_mx_meta_kernel<<<grid_for((int64_t)d->num_experts * L.nt * L.kb4 * 64, B), B, 0, s>>>(a);
  } else if (f == F_FP8_BLOCK) {
    repack_fp8_block_meta_kernel<<<grid_for((int64_t)d->num_experts * L.nt * L.kb, B), B, 0, s>>>(a);
  } else {
    repack_fp8_meta_kernel<<<grid_for((int64_t)d->num_experts * L.nt * kNSub, B), B, 0, s>>>(a);
  }
  repack_gscale_kernel<<<grid_for(d->num_experts, B), B, 0, s>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "repack launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

// ---------------------------------------------------------------------------
// Exact dequantization of the packed buffer: out[e][n][k] = (v - z) * S.

struct DequantArgs {
  const uint8_t* packed;
  float* out;
  int64_t n, k, nt, kb, ng, kb4, kb_per_group;
  int64_t codes_off, scales_off, zeros_off;
  int64_t codes_pe, scales_pe, zeros_pe;
  int num_experts, wdt, scale_f32, has_zero;
  int block;     // E4M3 with 2-D block scales
  int bf16_order;  // 8-bit codes in the bf16 MFMA order
  int nvfp4;       // E2M1 with E4M3 scales per 16
  int mxint4;      // INT4 with E8M0 scales per 32
};

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  float v = mag[c & 7];
  return (c & 8) ? -v : v;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  uint32_t s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  float v;
  if (e == 15 && m == 7) v = __uint_as_float(0x7FC00000u);
  else if (e == 0) v = (float)m * 0.001953125f;  // m * 2^-9
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return s ? -v : v;
}

__global__ void dequant_kernel(DequantArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.num_experts * a.nt * a.kb * 64;
  if (tid >= total) return;
  const int lane = (int)(tid & 63);
  int64_t rest = tid >> 6;
  const int64_t kb = rest % a.kb;
  rest /= a.kb;
  const int64_t nt = rest % a.nt;
  const int64_t e = rest / a.nt;
  const int c = lane & 15, lg = lane >> 4;
  const int64_t n = nt * kNSub + c;
  if (n >= a.n) return;
  const uint8_t* base = a.packed + a.codes_off + e * a.codes_pe;
  float* orow = a.out + (e * a.n + n) * a.k + kb * kKBlk;
  if (a.wdt == HUM_E4M3 || a.wdt == HUM_INT8) {
    const uint8_t* src = base + ((nt * a.kb + kb) * 64 + lane) * 32;
    const float* sp = reinterpret_cast<const float*>(a.packed + a.scales_off + e * a.scales_pe);
    const float s = a.block ? sp[nt * a.kb + kb] : sp[n];
    for (int j = 0; j < 32; ++j) {
      const int kk = a.bf16_order ? (32 * lg + j) : ((j < 16) ? (16 * lg + j) : (64 + 16 * lg + j - 16));
      orow[kk] = (a.wdt == HUM_INT8 ? (float)(int8_t)src[j] : e4m3_value(src[j])) * s;
    }
    return;
  }
  if (a.wdt == HUM_E2M3 || a.wdt == HUM_E3M2) {
    // FP6: sign, exponent (bias 1 / 3), mantissa; exponent 0 subnormal
    const uint32_t* w = reinterpret_cast<const uint32_t*>(base + ((nt * a.kb + kb) * 64 + lane) * 24);
    const uint32_t word = *reinterpret_cast<const uint32_t*>(
        a.packed + a.scales_off + e * a.scales_pe + ((nt * a.kb4 + kb / 4) * 64 + lane) * 4);
    const float s = e8m0_to_f32((word >> (8 * (kb % 4))) & 0xFF);
    const int eb = a.wdt == HUM_E2M3 ? 2 : 3, mb = 5 - eb, bias = a.wdt == HUM_E2M3 ? 1 : 3;
    for (int j = 0; j < 32; ++j) {
      const int bit = 6 * j;
      const uint64_t win = (uint64_t)w[bit / 32] | ((bit / 32 + 1 < 6) ? (uint64_t)w[bit / 32 + 1] << 32 : 0);
      const uint32_t c = (uint32_t)(win >> (bit % 32)) & 63u;
      const uint32_t ex = (c >> mb) & ((1u << eb) - 1), m = c & ((1u << mb) - 1);
      const float mag = ex == 0 ? ldexpf((float)m, 1 - bias - mb) : ldexpf(1.0f + ldexpf((float)m, -mb), (int)ex - bias);
      orow[32 * lg + j] = ((c & 32u) ? -mag : mag) * s;
    }
    return;
  }
  const int bits = dtype_int_bits(a.wdt);
  if (bits != 0 && bits < 4) {
    // b-bit integers: the bit planes of the lane's 32 codes
    const uint32_t* w = reinterpret_cast<const uint32_t*>(base + ((nt * a.kb + kb) * 64 + lane) * 4 * bits);
    const int64_t g = kb / a.kb_per_group;
    const uint8_t* sb = a.packed + a.scales_off + e * a.scales_pe;
    const float s = a.scale_f32 ? reinterpret_cast<const float*>(sb)[(nt * a.ng + g) * 16 + c]
                                : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(sb)[(nt * a.ng + g) * 16 + c]);
    int off = dtype_int_signed(a.wdt) ? (1 << (bits - 1)) : 0;
    if (a.has_zero) {
      const uint64_t zp = *reinterpret_cast<const uint64_t*>(a.packed + a.zeros_off + e * a.zeros_pe + (nt * a.ng + g) * 8);
      off += (int)((zp >> (4 * c)) & 0xF);
    }
    for (int st = 0; st < 4; ++st)
      for (int j = 0; j < 8; ++j) {
        uint32_t u = 0;
        if (bits >= 2) u = (w[st >> 1] >> ((j & 1) * 16 + 2 * (4 * (st & 1) + (j >> 1)))) & 3u;
        if (bits != 2) {
          const uint32_t b1 = (w[bits == 3 ? 2 : 0] >> ((j & 1) * 16 + 4 * st + (j >> 1))) & 1u;
          u |= bits == 3 ? (b1 << 2) : b1;
        }
        orow[32 * lg + 8 * st + j] = (float)((int)u - off) * s;
      }
    return;
  }
  const u32x4_t w = *reinterpret_cast<const u32x4_t*>(base + ((nt * a.kb + kb) * 64 + lane) * 16);
  if (a.wdt == HUM_E2M1 && a.nvfp4) {
    const uint32_t word = *reinterpret_cast<const uint32_t*>(
        a.packed + a.scales_off + e * a.scales_pe + ((nt * a.kb4 + kb / 2) * 64 + lane) * 4);
    for (int j = 0; j < 32; ++j) {
      const uint32_t code = (w[j / 8] >> (4 * (j % 8))) & 0xF;
      const float s = e4m3_value((word >> (8 * (2 * (kb % 2) + j / 16))) & 0xFF);
      orow[32 * lg + j] = e2m1_value(code) * s;
    }
    return;
  }
  if (a.wdt == HUM_E2M1) {
    const uint32_t word = *reinterpret_cast<const uint32_t*>(
        a.packed + a.scales_off + e * a.scales_pe + ((nt * a.kb4 + kb / 4) * 64 + lane) * 4);
    const float s = e8m0_to_f32((word >> (8 * (kb % 4))) & 0xFF);
    for (int j = 0; j < 32; ++j) {
      const uint32_t code = (w[j / 8] >> (4 * (j % 8))) & 0xF;
      orow[32 * lg + j] = e2m1_value(code) * s;
    }
    return;
  }
  if (a.mxint4) {
    // INT4 codes in the integer nibble order (stored q + 8), E8M0 per 32
    const uint32_t word = *reinterpret_cast<const uint32_t*>(
        a.packed + a.scales_off + e * a.scales_pe + ((nt * a.kb4 + kb / 4) * 64 + lane) * 4);
    const float s = e8m0_to_f32((word >> (8 * (kb % 4))) & 0xFF);
    for (int st = 0; st < 4; ++st)
      for (int j = 0; j < 8; ++j) {
        const uint32_t u = (w[st] >> ((j & 1) * 16 + (j >> 1) * 4)) & 0xF;
        orow[32 * lg + 8 * st + j] = (float)((int)u - 8) * s;
      }
    return;
  }
  // INT4 / UINT4
  const int64_t g = kb / a.kb_per_group;
  const uint8_t* sb = a.packed + a.scales_off + e * a.scales_pe;
  const float s = a.scale_f32 ? reinterpret_cast<const float*>(sb)[(nt * a.ng + g) * 16 + c]
                              : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(sb)[(nt * a.ng + g) * 16 + c]);
  int off = (a.wdt == HUM_INT4) ? 8 : 0;
  if (a.has_zero) {
    const uint64_t zp = *reinterpret_cast<const uint64_t*>(a.packed + a.zeros_off + e * a.zeros_pe + (nt * a.ng + g) * 8);
    off += (int)((zp >> (4 * c)) & 0xF);
  }
  for (int st = 0; st < 4; ++st) {
    for (int j = 0; j < 8; ++j) {
      const uint32_t u = (w[st] >> ((j & 1) * 16 + (j >> 1) * 4)) & 0xF;
      orow[32 * lg + 8 * st + j] = (float)((int)u - off) * s;
    }
  }
}

hum_status launch_dequant(const hum_weight_desc* d, const Layout& L, const void* packed,
                          float* out, void* stream) {
  DequantArgs a;
  a.packed = static_cast<const uint8_t*>(packed);
  a.out = out;
  a.n = d->n;
  a.k = d->k;
  a.nt = L.nt;
  a.kb = L.kb;
  a.ng = L.ng;
  a.kb4 = L.kb4;
  a.kb_per_group = L.kb_per_group;
  a.codes_off = L.codes_off;
  a.scales_off = L.scales_off;
  a.zeros_off = L.zeros_off;
  a.codes_pe = L.codes_per_expert;
  a.scales_pe = L.scales_per_expert;
  a.zeros_pe = L.zeros_per_expert;
  a.num_experts = d->num_experts;
  a.wdt = d->weight_dtype;
  a.scale_f32 = L.scale_f32;
  a.has_zero = d->has_zero_point;
  a.block = d->scale_gran == HUM_SCALE_BLOCK;
  a.bf16_order = fmt_w8_bf16(fmt_of(d));
  a.nvfp4 = fmt_of(d) == F_NVFP4_BF16;
  a.mxint4 = fmt_of(d) == F_MXINT4_BF16;
  const int64_t total = (int64_t)d->num_experts * L.nt * L.kb * 64;
  dequant_kernel<<<grid_for(total, 256), 256, 0, static_cast<hipStream_t>(stream)>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "dequant launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

}  // namespace hum
