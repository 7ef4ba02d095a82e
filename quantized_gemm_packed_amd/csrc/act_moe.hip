// Activation quantizers, MoE routing align and the top-k weighted reduce.
//
// * Activation formats: "tokenwise FP8" (Announcing Humming, section
//   "End-to-end inference performance") and MXFP8 (section "Choosing the
//   activation type"); scale rules are the OCP ones (see hum.h).
// * Align = "moe_align_block_size" / "moe_permute_prepare" and reduce =
//   "moe_fused_mul_sum" of the SGLang PR #23754 summary ("Implementation
//   breakdown", "Review highlights").  Both are written for gfx950 here: one
//   workgroup sorts by expert with wave ballots (stable, no atomics on the
//   output order), and the reduce streams 16-byte rows.
#include "dev_common.h"
#include "hum_internal.h"

namespace hum {

static inline unsigned cdiv_u(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

// ---------------------------------------------------------------------------
// Per-token FP8: one workgroup per row.

__global__ __launch_bounds__(256) void quant_fp8_token_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                              int64_t k, uint8_t* __restrict__ q,
                                                              float* __restrict__ s,
                                                              const int32_t* __restrict__ sorted, int32_t sentinel) {
  const int64_t row = blockIdx.x;
  if (sorted && sorted[row] >= sentinel) return;  // a padding slot of grouped rows
  const uint16_t* xr = x + row * ldx;
  const int tid = threadIdx.x;
  __shared__ float red[4];
  float amax = 0.0f;
  for (int64_t c = (int64_t)tid * 8; c < k; c += 256 * 8) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(xr + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      amax = __builtin_fmaxf(amax, __builtin_fabsf(bf16_bits_to_f32(v[i] & 0xFFFF)));
      amax = __builtin_fmaxf(amax, __builtin_fabsf(bf16_bits_to_f32(v[i] >> 16)));
    }
  }
  amax = row16_max(amax);
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;  // IEEE f32 division
  if (tid == 0) s[row] = sc;
  uint8_t* qr = q + row * k;
  for (int64_t c = (int64_t)tid * 8; c < k; c += 256 * 8) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(xr + c);
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_bits_to_f32(v[i] & 0xFFFF) / sc;
      const float b = bf16_bits_to_f32(v[i] >> 16) / sc;
      const uint32_t p = f32x2_to_e4m3x2(a, b);
      if (i < 2) w0 |= p << (16 * i);
      else w1 |= p << (16 * (i - 2));
    }
    uint2 o;
    o.x = w0;
    o.y = w1;
    *reinterpret_cast<uint2*>(qr + c) = o;
  }
}

hum_status launch_quant_fp8_token(int64_t m, int64_t k, const void* x, int64_t ldx, void* q,
                                  float* s, void* stream, const int32_t* sorted, int32_t sentinel) {
  if (m == 0) return HUM_OK;
  quant_fp8_token_kernel<<<(unsigned)m, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint16_t*>(x), ldx, k, static_cast<uint8_t*>(q), s, sorted, sentinel);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "quant_fp8_token launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

// ---------------------------------------------------------------------------
// Per-token-group FP8 (groups of 128 along K): each thread quantizes 8
// elements; a DPP row of 16 lanes owns one group.  The per-token rule per
// group: s = amax / 448 (IEEE f32 division; 1 for an all-zero group),
// q = E4M3_RNE_SAT(x / s).

__global__ __launch_bounds__(256) void quant_fp8_group_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                              int64_t m, int64_t k, uint8_t* __restrict__ q,
                                                              float* __restrict__ s,
                                                              const int32_t* __restrict__ sorted, int32_t sentinel) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t cpr = k / 8;  // chunks per row
  // (a padding slot of grouped rows is skipped: its 16-lane groups all
  // belong to the one row, so they drop out together)
  const bool valid = id < m * cpr && !(sorted && sorted[id / cpr] >= sentinel);
  const int64_t row = valid ? id / cpr : 0;
  const int64_t c8 = valid ? id % cpr : 0;
  u32x4_t v = {0, 0, 0, 0};
  if (valid) v = *reinterpret_cast<const u32x4_t*>(x + row * ldx + c8 * 8);
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_bits_to_f32(v[i] & 0xFFFF);
    f[2 * i + 1] = bf16_bits_to_f32(v[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
  amax = row16_max(amax);  // the 16 chunks of one 128-group are one DPP row
  const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (!valid) return;
  uint2 o;
  o.x = f32x2_to_e4m3x2(f[0] / sc, f[1] / sc) | (f32x2_to_e4m3x2(f[2] / sc, f[3] / sc) << 16);
  o.y = f32x2_to_e4m3x2(f[4] / sc, f[5] / sc) | (f32x2_to_e4m3x2(f[6] / sc, f[7] / sc) << 16);
  *reinterpret_cast<uint2*>(q + row * k + c8 * 8) = o;
  if ((c8 & 15) == 0) s[row * (k / 128) + c8 / 16] = sc;
}

hum_status launch_quant_fp8_group(int64_t m, int64_t k, const void* x, int64_t ldx, void* q, float* s,
                                  void* stream, const int32_t* sorted, int32_t sentinel) {
  if (m == 0) return HUM_OK;
  const int64_t chunks = m * (k / 8);
  quant_fp8_group_kernel<<<cdiv_u(chunks, 256), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint16_t*>(x), ldx, m, k, static_cast<uint8_t*>(q), s, sorted, sentinel);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "quant_fp8_group launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

// ---------------------------------------------------------------------------
// MXFP8: each thread quantizes 8 elements; a DPP quad owns one 32-block.

// One 8-element chunk (row, c8) of the MXFP8 quantizer; every lane of a
// wave calls it together (the DPP quad reduction reads the quad's four
// lanes), with valid = false for lanes that have no chunk.
__device__ __forceinline__ void mxfp8_chunk(const uint16_t* __restrict__ x, int64_t ldx, int64_t k, int64_t row,
                                              int64_t c8, bool valid, uint8_t* __restrict__ q,
                                              uint8_t* __restrict__ s) {
  u32x4_t v = {0, 0, 0, 0};
  if (valid) v = *reinterpret_cast<const u32x4_t*>(x + row * ldx + c8 * 8);
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_bits_to_f32(v[i] & 0xFFFF);
    f[2 * i + 1] = bf16_bits_to_f32(v[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
  amax = quad_max(amax);  // the 4 chunks of one 32-block are one DPP quad
  const int e = mx_scale_code(amax);
  const float inv = mx_inv_scale(e);
  if (!valid) return;
  uint2 o;
  o.x = f32x2_to_e4m3x2(f[0] * inv, f[1] * inv) | (f32x2_to_e4m3x2(f[2] * inv, f[3] * inv) << 16);
  o.y = f32x2_to_e4m3x2(f[4] * inv, f[5] * inv) | (f32x2_to_e4m3x2(f[6] * inv, f[7] * inv) << 16);
  *reinterpret_cast<uint2*>(q + row * k + c8 * 8) = o;
  if ((c8 & 3) == 0) s[row * (k / 32) + c8 / 4] = (uint8_t)e;
}

__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                          int64_t m, int64_t k, uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ s) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t cpr = k / 8;  // chunks per row
  const bool valid = id < m * cpr;
  mxfp8_chunk(x, ldx, k, valid ? id / cpr : 0, valid ? id % cpr : 0, valid, q, s);
}

// grouped_masked buffers: workgroup (e, slice) walks rows slice, slice +
// slices, ... below expert e's count (clamped to [0, max_m]); rows past
// it are not read.  Loop bounds are uniform over the workgroup.
__global__ __launch_bounds__(256) void quant_mxfp8_masked_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                                 int64_t k, const int32_t* __restrict__ counts,
                                                                 int64_t max_m, int slices,
                                                                 uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int64_t e = blockIdx.x / slices;
  const int slice = (int)(blockIdx.x % slices);
  int64_t c = counts[e];
  c = c < 0 ? 0 : (c > max_m ? max_m : c);
  const int64_t cpr = k / 8;
  for (int64_t i = slice; i < c; i += slices)
    for (int64_t base = 0; base < cpr; base += 256) {
      const int64_t c8 = base + threadIdx.x;
      mxfp8_chunk(x, ldx, k, e * max_m + i, c8 < cpr ? c8 : 0, c8 < cpr, q, s);
    }
}

hum_status launch_quant_mxfp8(int64_t m, int64_t k, const void* x, int64_t ldx, void* q,
                              uint8_t* s, void* stream, const int32_t* counts, int64_t max_m) {
  if (m == 0) return HUM_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (counts) {
    // m = E * max_m rows; about 2048 workgroups over the experts
    const int64_t e = m / max_m;
    const int slices = (int)(e >= 2048 ? 1 : (2048 + e - 1) / e);
    quant_mxfp8_masked_kernel<<<(unsigned)(e * slices), 256, 0, st>>>(
        static_cast<const uint16_t*>(x), ldx, k, counts, max_m, slices, static_cast<uint8_t*>(q), s);
  } else {
    const int64_t chunks = m * (k / 8);
    quant_mxfp8_kernel<<<cdiv_u(chunks, 256), 256, 0, st>>>(static_cast<const uint16_t*>(x), ldx, m, k,
                                                              static_cast<uint8_t*>(q), s);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "quant_mxfp8 launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

// ---------------------------------------------------------------------------
// MXFP4: each thread quantizes 8 elements into 4 bytes of E2M1 pairs (even k
// in the low nibble); a DPP quad owns one 32-block.  The block scale follows
// the MXFP8 rule with E2M1's emax (2); x / 2^(E-127) is exact in f32 (a
// power-of-two scaling of a bf16 value, at most 8 in magnitude; results
// below f32's range round to 0 in E2M1 either way), and the rounding to the
// E2M1 grid is a comparison against the midpoints, ties to the even code.


// One 8-element chunk (row, c8) of the MXFP4 quantizer; every lane of a
// wave calls it together (the DPP quad reduction reads the quad's four
// lanes), with valid = false for lanes that have no chunk.
// WIDE: each E2M1 code is written as the E4M3 byte of the same value (one
// byte per element, k bytes per row), for the E4M3 x E2M1 decode kernel: an
// MXFP4 activation block is then an MXFP8 block with the same E8M0 scale.
template <bool WIDE = false>
__device__ __forceinline__ void mxfp4_chunk(const uint16_t* __restrict__ x, int64_t ldx, int64_t k, int64_t row,
                                              int64_t c8, bool valid, uint8_t* __restrict__ q,
                                              uint8_t* __restrict__ s) {
  u32x4_t v = {0, 0, 0, 0};
  if (valid) v = *reinterpret_cast<const u32x4_t*>(x + row * ldx + c8 * 8);
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_bits_to_f32(v[i] & 0xFFFF);
    f[2 * i + 1] = bf16_bits_to_f32(v[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
  amax = quad_max(amax);  // the 4 chunks of one 32-block are one DPP quad
  const int e = mx_scale_code_emax(amax, 2);
  const float inv = mx_inv_scale(e);
  if (!valid) return;
  if constexpr (WIDE) {
    // E2M1 magnitude code -> E4M3 byte: 0, 0.5, 1, 1.5, 2, 3, 4, 6
    constexpr uint64_t kE4m3Of = 0x4C4844403C383000ull;
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = f32_to_e2m1(f[i] * inv);
      const uint32_t b = (uint32_t)((kE4m3Of >> (8 * (c & 7))) & 0xFF) | ((c & 8) << 4);
      o[i >> 2] |= b << (8 * (i & 3));
    }
    *reinterpret_cast<uint2*>(q + row * k + c8 * 8) = make_uint2(o[0], o[1]);
  } else {
    uint32_t o = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) o |= f32_to_e2m1(f[i] * inv) << (4 * i);
    *reinterpret_cast<uint32_t*>(q + row * (k / 2) + c8 * 4) = o;
  }
  if ((c8 & 3) == 0) s[row * (k / 32) + c8 / 4] = (uint8_t)e;
}

template <bool WIDE>
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                          int64_t m, int64_t k, uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ s) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t cpr = k / 8;  // chunks per row
  const bool valid = id < m * cpr;
  mxfp4_chunk<WIDE>(x, ldx, k, valid ? id / cpr : 0, valid ? id % cpr : 0, valid, q, s);
}

// grouped_masked buffers: workgroup (e, slice) walks rows slice, slice +
// slices, ... below expert e's count (clamped to [0, max_m]); rows past
// it are not read.  Loop bounds are uniform over the workgroup.
__global__ __launch_bounds__(256) void quant_mxfp4_masked_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                                 int64_t k, const int32_t* __restrict__ counts,
                                                                 int64_t max_m, int slices,
                                                                 uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int64_t e = blockIdx.x / slices;
  const int slice = (int)(blockIdx.x % slices);
  int64_t c = counts[e];
  c = c < 0 ? 0 : (c > max_m ? max_m : c);
  const int64_t cpr = k / 8;
  for (int64_t i = slice; i < c; i += slices)
    for (int64_t base = 0; base < cpr; base += 256) {
      const int64_t c8 = base + threadIdx.x;
      mxfp4_chunk(x, ldx, k, e * max_m + i, c8 < cpr ? c8 : 0, c8 < cpr, q, s);
    }
}

hum_status launch_quant_mxfp4(int64_t m, int64_t k, const void* x, int64_t ldx, void* q,
                              uint8_t* s, void* stream, const int32_t* counts, int64_t max_m) {
  if (m == 0) return HUM_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (counts) {
    // m = E * max_m rows; about 2048 workgroups over the experts
    const int64_t e = m / max_m;
    const int slices = (int)(e >= 2048 ? 1 : (2048 + e - 1) / e);
    quant_mxfp4_masked_kernel<<<(unsigned)(e * slices), 256, 0, st>>>(
        static_cast<const uint16_t*>(x), ldx, k, counts, max_m, slices, static_cast<uint8_t*>(q), s);
  } else {
    const int64_t chunks = m * (k / 8);
    quant_mxfp4_kernel<false><<<cdiv_u(chunks, 256), 256, 0, st>>>(static_cast<const uint16_t*>(x), ldx, m, k,
                                                                     static_cast<uint8_t*>(q), s);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "quant_mxfp4 launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

hum_status launch_quant_mxfp4_wide(int64_t m, int64_t k, const void* x, int64_t ldx, void* q, uint8_t* s,
                                   void* stream) {
  if (m == 0) return HUM_OK;
  const int64_t chunks = m * (k / 8);
  quant_mxfp4_kernel<true><<<cdiv_u(chunks, 256), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint16_t*>(x), ldx, m, k, static_cast<uint8_t*>(q), s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "quant_mxfp4 (E4M3 bytes) launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

// ---------------------------------------------------------------------------
// Fill kernel (used instead of hipMemsetAsync so the path stays capturable).

__global__ void zero_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

hum_status launch_zero(void* p, size_t bytes, void* stream) {
  const int64_t words = (int64_t)(bytes / 4);
  if (words == 0) return HUM_OK;
  int64_t g = (words + 255) / 256;
  if (g > 4096) g = 4096;
  zero_kernel<<<(unsigned)g, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<uint32_t*>(p), words);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "zero launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

// ---------------------------------------------------------------------------
// Align: stable counting sort of the flat slots f = t*topk + j by expert,
// segments padded to block_m, plus the block -> expert map of the GEMMs.

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;
constexpr int kMaxExperts = 512;
static_assert(kAlignThreads >= kMaxExperts, "one thread per expert in the offset scan");

// Stable scatter of ids [i0, i1) (one workgroup, kAlignThreads lanes):
// running[e] holds the next position of expert e's slots.  Sub-chunks of
// kAlignThreads slots; lanes of a wave holding the same expert are found
// with one ballot per id bit, per-wave counts go through an LDS table, so a
// slot's position is running[e] + earlier waves + earlier lanes.
__device__ void align_scatter_range(const int32_t* __restrict__ ids, int64_t i0, int64_t i1, int32_t E,
                                    int32_t* running, int32_t (*wcnt)[kMaxExperts],
                                    int32_t* __restrict__ sorted) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int nbits = 1;
  while ((1 << nbits) <= E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t base = i0; base < i1; base += kAlignThreads) {
    const int64_t i = base + tid;
    int32_t e = (i < i1) ? ids[i] : -1;
    if (e < 0 || e >= E) e = -1;
    const uint32_t key = (uint32_t)(e + 1);
    uint64_t same = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1u;
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int rank_w = __popcll(same & lt_mask);
    const bool leader = (same & lt_mask) == 0;
    for (int idx = tid; idx < kAlignWaves * E; idx += kAlignThreads) wcnt[idx / E][idx % E] = 0;
    __syncthreads();
    if (leader && e >= 0) wcnt[wave][e] = __popcll(same);
    __syncthreads();
    if (e >= 0) {
      int32_t prefix = 0;
      for (int w = 0; w < wave; ++w) prefix += wcnt[w][e];
      sorted[running[e] + prefix + rank_w] = (int32_t)i;
    }
    __syncthreads();
    for (int ex = tid; ex < E; ex += kAlignThreads) {
      int32_t tot = 0;
      for (int w = 0; w < kAlignWaves; ++w) tot += wcnt[w][ex];
      running[ex] += tot;
    }
    __syncthreads();
  }
}

// Padded segment offsets from per-expert counts (one workgroup): off[e+1] =
// off[e] + ceil(cnt[e] / block_m) * block_m, a shuffle scan inside each wave
// (64 experts), then the wave totals.
__device__ void align_offsets(const int32_t* cnt, int32_t E, int32_t block_m, int32_t* off) {
  __shared__ int32_t wsum[kMaxExperts / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int e = tid;
  int32_t v = 0;
  if (e < E) v = (cnt[e] + block_m - 1) / block_m * block_m;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  if (e < kMaxExperts && lane == 63) wsum[wave] = v;
  __syncthreads();
  if (e < E) {
    int32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    off[e + 1] = before + v;
  }
  if (tid == 0) off[0] = 0;
  __syncthreads();
}

// The block -> expert map (block b: rows b*block_m ..; -1 past off[E]).
__device__ void align_block_experts(const int32_t* off, int32_t E, int32_t block_m, int32_t* __restrict__ block_expert,
                                    int64_t nblocks) {
  for (int64_t b = threadIdx.x; b < nblocks; b += kAlignThreads) {
    const int64_t pos = b * block_m;
    int32_t ex = -1;
    if (pos < off[E]) {
      int lo = 0, hi = E - 1;  // largest e with off[e] <= pos
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= pos) lo = mid;
        else hi = mid - 1;
      }
      ex = lo;
    }
    block_expert[b] = ex;
  }
}

// One workgroup for the whole sort (small routing tables).
__global__ __launch_bounds__(kAlignThreads) void align_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                              int32_t num_experts, int32_t block_m,
                                                              int32_t* __restrict__ sorted, int64_t cap,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ block_expert,
                                                              int64_t nblocks) {
  __shared__ int32_t cnt[kMaxExperts];
  __shared__ int32_t off[kMaxExperts + 1];
  __shared__ int32_t running[kMaxExperts];
  __shared__ int32_t wcnt[kAlignWaves][kMaxExperts];  // per-wave counts of one sub-chunk
  const int tid = threadIdx.x;
  const int32_t E = num_experts;
  const int32_t sentinel = (int32_t)n;
  for (int64_t i = tid; i < cap; i += kAlignThreads) sorted[i] = sentinel;
  for (int e = tid; e < E; e += kAlignThreads) cnt[e] = 0;
  __syncthreads();
  for (int64_t i = tid; i < n; i += kAlignThreads) {
    const int32_t e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  align_offsets(cnt, E, block_m, off);
  for (int e = tid; e <= E; e += kAlignThreads) offsets[e] = off[e];
  for (int e = tid; e < E; e += kAlignThreads) {
    counts[e] = cnt[e];
    running[e] = off[e];
  }
  align_block_experts(off, E, block_m, block_expert, nblocks);
  __syncthreads();
  align_scatter_range(ids, 0, n, E, running, wcnt, sorted);
}

// One wave for routing tables of at most 64 slots (decode batches): lane f
// holds slot f.  The lanes of one expert find each other with one ballot per
// id bit; a slot's place in its expert's segment is the number of earlier
// lanes of that expert (the stable order), and the expert's first lane (its
// leader) owns the rest of the segment: its padding and its blocks of the
// block -> expert map.  Every sorted entry and map entry is written exactly
// once, so no store needs ordering against another.
constexpr int kAlignSmall = 64;

__global__ __launch_bounds__(64) void align_small_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                         int32_t num_experts, int32_t block_m,
                                                         int32_t* __restrict__ sorted, int64_t cap,
                                                         int32_t* __restrict__ offsets, int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ block_expert, int64_t nblocks) {
  __shared__ int32_t cnt[kMaxExperts];
  __shared__ int32_t off[kMaxExperts];
  const int lane = threadIdx.x;
  const int32_t E = num_experts;
  const int32_t sentinel = (int32_t)n;
  int32_t e = lane < n ? ids[lane] : -1;
  if (e < 0 || e >= E) e = -1;
  for (int x = lane; x < E; x += 64) cnt[x] = 0;
  int nbits = 1;
  while ((1 << nbits) <= E) ++nbits;
  const uint32_t key = (uint32_t)(e + 1);
  uint64_t same = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t bal = __ballot(bit);
    same &= bit ? bal : ~bal;
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(same & lt_mask);
  const int c = __popcll(same);
  const bool leader = e >= 0 && rank == 0;
  __syncthreads();
  if (leader) cnt[e] = c;
  __syncthreads();
  // padded offsets: lane l scans experts [l * per, (l + 1) * per)
  const int per = (E + 63) / 64;
  int32_t s = 0;
  for (int i = 0; i < per; ++i) {
    const int x = lane * per + i;
    if (x < E) s += (cnt[x] + block_m - 1) / block_m * block_m;
  }
  int32_t inc = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t u = __shfl_up(inc, d);
    if (lane >= d) inc += u;
  }
  const int32_t total = __shfl(inc, 63);
  int32_t run = inc - s;
  for (int i = 0; i < per; ++i) {
    const int x = lane * per + i;
    if (x < E) {
      off[x] = run;
      offsets[x] = run;
      counts[x] = cnt[x];
      run += (cnt[x] + block_m - 1) / block_m * block_m;
    }
  }
  if (lane == 0) offsets[E] = total;
  __syncthreads();
  if (e >= 0) sorted[off[e] + rank] = lane;
  if (leader) {
    const int32_t o = off[e];
    const int32_t psz = (c + block_m - 1) / block_m * block_m;
    for (int32_t r = c; r < psz; ++r) sorted[o + r] = sentinel;
    if (block_expert)
      for (int32_t q = 0; q < psz / block_m; ++q)
        if (o / block_m + q < nblocks) block_expert[o / block_m + q] = e;
  }
  for (int64_t i = total + lane; i < cap; i += 64) sorted[i] = sentinel;
  if (block_expert)
    for (int64_t b = total / block_m + lane; b < nblocks; b += 64) block_expert[b] = -1;
}

// Multi-workgroup sort (large routing tables), three launches:
//   count   : workgroup g counts the experts of ids [g C, (g+1) C) -> part[g][e]
//   scan    : one workgroup: totals, padded offsets, and part[g][e] becomes
//             the position of chunk g's first slot of expert e (offset of e
//             plus the counts of the chunks before g); sentinel fill, block map
//   scatter : workgroup g places its chunk's slots from part[g][e] on
// The result is the same stable order as the one-workgroup sort.
constexpr int64_t kAlignChunk = 4096;

__global__ __launch_bounds__(kAlignThreads) void align_count_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                                    int32_t E, int32_t* __restrict__ part) {
  __shared__ int32_t cnt[kMaxExperts];
  const int tid = threadIdx.x;
  const int64_t i0 = (int64_t)blockIdx.x * kAlignChunk;
  const int64_t i1 = i0 + kAlignChunk < n ? i0 + kAlignChunk : n;
  for (int e = tid; e < E; e += kAlignThreads) cnt[e] = 0;
  __syncthreads();
  for (int64_t i = i0 + tid; i < i1; i += kAlignThreads) {
    const int32_t e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kAlignThreads) part[(int64_t)blockIdx.x * E + e] = cnt[e];
}

__global__ __launch_bounds__(kAlignThreads) void align_scan_kernel(int32_t* __restrict__ part, int64_t chunks,
                                                                   int64_t n, int32_t E, int32_t block_m,
                                                                   int32_t* __restrict__ sorted, int64_t cap,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ block_expert,
                                                                   int64_t nblocks) {
  __shared__ int32_t cnt[kMaxExperts];
  __shared__ int32_t off[kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int32_t sentinel = (int32_t)n;
  for (int64_t i = tid; i < cap; i += kAlignThreads) sorted[i] = sentinel;
  // per expert: running sums over the chunks (counts before chunk g)
  for (int e = tid; e < E; e += kAlignThreads) {
    int32_t run = 0;
    for (int64_t g = 0; g < chunks; ++g) {
      const int32_t c = part[g * E + e];
      part[g * E + e] = run;
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();
  align_offsets(cnt, E, block_m, off);
  for (int e = tid; e <= E; e += kAlignThreads) offsets[e] = off[e];
  for (int e = tid; e < E; e += kAlignThreads) {
    counts[e] = cnt[e];
    for (int64_t g = 0; g < chunks; ++g) part[g * E + e] += off[e];
  }
  align_block_experts(off, E, block_m, block_expert, nblocks);
}

__global__ __launch_bounds__(kAlignThreads) void align_scatter_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                                      int32_t E, const int32_t* __restrict__ part,
                                                                      int32_t* __restrict__ sorted) {
  __shared__ int32_t running[kMaxExperts];
  __shared__ int32_t wcnt[kAlignWaves][kMaxExperts];
  const int64_t i0 = (int64_t)blockIdx.x * kAlignChunk;
  const int64_t i1 = i0 + kAlignChunk < n ? i0 + kAlignChunk : n;
  for (int e = threadIdx.x; e < E; e += kAlignThreads) running[e] = part[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  align_scatter_range(ids, i0, i1, E, running, wcnt, sorted);
}

int64_t align_workspace_bytes(int64_t t, int32_t topk, int32_t e) {
  const int64_t n = t * topk;
  return n > kAlignChunk ? ((n + kAlignChunk - 1) / kAlignChunk) * (int64_t)e * 4 : 0;
}

hum_status launch_align(const int32_t* ids, int64_t t, int32_t topk, int32_t e, int32_t block_m,
                        int32_t* sorted, int32_t* offsets, int32_t* counts, int32_t* block_expert,
                        int64_t nblocks, void* stream, void* tmp, int64_t tmp_bytes) {
  if (e > kMaxExperts) return set_error(HUM_ERR_UNSUPPORTED, "align: at most %d experts", kMaxExperts);
  const int64_t n = t * topk;
  const int64_t cap = n + (int64_t)e * (block_m - 1);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t need = align_workspace_bytes(t, topk, e);
  if (need > 0 && tmp && tmp_bytes >= need) {
    const int64_t chunks = (n + kAlignChunk - 1) / kAlignChunk;
    int32_t* part = static_cast<int32_t*>(tmp);
    align_count_kernel<<<(unsigned)chunks, kAlignThreads, 0, s>>>(ids, n, e, part);
    align_scan_kernel<<<1, kAlignThreads, 0, s>>>(part, chunks, n, e, block_m, sorted, cap, offsets, counts,
                                                  block_expert, nblocks);
    align_scatter_kernel<<<(unsigned)chunks, kAlignThreads, 0, s>>>(ids, n, e, part, sorted);
  } else if (n <= kAlignSmall) {
    align_small_kernel<<<1, 64, 0, s>>>(ids, n, e, block_m, sorted, cap, offsets, counts, block_expert, nblocks);
  } else {
    align_kernel<<<1, kAlignThreads, 0, s>>>(ids, n, e, block_m, sorted, cap, offsets, counts, block_expert,
                                             nblocks);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "align launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

// ---------------------------------------------------------------------------
// Reduce: out[t][:] = bf16(sum_j w[t][j] * y[t*topk + j][:]), fp32, j order.

__global__ __launch_bounds__(256) void moe_reduce_kernel(const uint16_t* __restrict__ y, const float* __restrict__ w,
                                                         const int32_t* __restrict__ ids, int32_t num_experts,
                                                         int64_t t_count, int32_t topk, int64_t h,
                                                         uint16_t* __restrict__ out) {
  const int64_t cpr = h / 8;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= t_count * cpr) return;
  const int64_t t = id / cpr, c8 = id % cpr;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  // Slots in chunks of 8: every load of a chunk (ids, weights, y rows) is
  // issued before any is used, so a chunk costs one memory latency, not one
  // per slot.  The y row of every existing slot is in bounds; a slot routed
  // outside [0, E) (an expert held elsewhere) was never computed and its
  // stale row is skipped, not multiplied by zero.
  for (int j0 = 0; j0 < topk; j0 += 8) {
    int32_t e[8];
    float wj[8];
    u32x4_t v[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = j0 + jj < topk ? j0 + jj : topk - 1;
      const int64_t f = t * topk + j;
      e[jj] = ids ? ids[f] : 0;
      wj[jj] = w[f];
      v[jj] = *reinterpret_cast<const u32x4_t*>(y + f * h + c8 * 8);
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (j0 + jj >= topk || (ids && (e[jj] < 0 || e[jj] >= num_experts))) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += wj[jj] * bf16_bits_to_f32(v[jj][i] & 0xFFFF);
        acc[2 * i + 1] += wj[jj] * bf16_bits_to_f32(v[jj][i] >> 16);
      }
    }
  }
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16_bits(acc[2 * i]) | (f32_to_bf16_bits(acc[2 * i + 1]) << 16);
  *reinterpret_cast<u32x4_t*>(out + t * h + c8 * 8) = o;
}

hum_status launch_moe_reduce(const void* y, const float* w, int64_t t, int32_t topk, int64_t h,
                             void* out, void* stream, const int32_t* ids, int32_t num_experts) {
  if (t == 0) return HUM_OK;
  moe_reduce_kernel<<<cdiv_u(t * (h / 8), 256), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint16_t*>(y), w, ids, num_experts, t, topk, h, static_cast<uint16_t*>(out));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "moe_reduce launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

// ---------------------------------------------------------------------------
// Block -> expert map of grouped rows from align's padded offsets: block b
// (rows b*block_m ..) belongs to the largest e with offsets[e] <= b*block_m,
// or to none (-1) past offsets[E].

__global__ void block_expert_kernel(const int32_t* __restrict__ offsets, int32_t num_experts, int32_t block_m,
                                    int64_t nblocks, int32_t* __restrict__ block_expert) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const int64_t pos = b * block_m;
  int32_t ex = -1;
  if (pos < offsets[num_experts]) {
    int lo = 0, hi = num_experts - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (offsets[mid] <= pos) lo = mid;
      else hi = mid - 1;
    }
    ex = lo;
  }
  block_expert[b] = ex;
}

hum_status launch_block_expert(const int32_t* offsets, int32_t e, int32_t block_m, int64_t nblocks,
                               int32_t* block_expert, void* stream) {
  if (nblocks == 0) return HUM_OK;
  block_expert_kernel<<<cdiv_u(nblocks, 256), 256, 0, static_cast<hipStream_t>(stream)>>>(offsets, e, block_m,
                                                                                           nblocks, block_expert);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "block_expert launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

// ---------------------------------------------------------------------------
// grouped_masked layout: one thread per row position (and per block).

__global__ void masked_align_kernel(const int32_t* __restrict__ counts, int32_t num_experts, int64_t max_m,
                                    int32_t block_m, int32_t* __restrict__ sorted,
                                    int32_t* __restrict__ block_expert) {
  const int64_t total = (int64_t)num_experts * max_m;
  const int64_t pos = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (pos >= total) return;
  const int64_t e = pos / max_m;
  const int64_t i = pos - e * max_m;
  int64_t c = counts[e];
  c = c < 0 ? 0 : (c > max_m ? max_m : c);
  sorted[pos] = i < c ? (int32_t)pos : (int32_t)total;
  if (i % block_m == 0) block_expert[pos / block_m] = i < c ? (int32_t)e : -1;
}

hum_status launch_masked_align(const int32_t* counts, int32_t e, int64_t max_m, int32_t block_m,
                               int32_t* sorted, int32_t* block_expert, void* stream) {
  const int64_t total = (int64_t)e * max_m;
  if (total == 0) return HUM_OK;
  const int B = 256;
  masked_align_kernel<<<(unsigned)((total + B - 1) / B), B, 0, static_cast<hipStream_t>(stream)>>>(
      counts, e, max_m, block_m, sorted, block_expert);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "masked align launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

}  // namespace hum
