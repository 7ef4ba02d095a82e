// Quantized GEMM for gfx950: dense layers and grouped (MoE) expert layers.
//
// What is computed is the WnA16 / W8A8 / W4A8 GEMM of "Announcing Humming:
// Fast, Flexible Kernels for Quantized Inference" (sections "WnA16" and
// "W8A8 / W4A8 / W4A4"): dequantization and scaling fused into the GEMM
// (section "Shared CUDA components"), per-GEMM-type task mapping for dense and
// MoE work, scale / bias epilogues.  The design is gfx950's own:
//
// * One workgroup = 4 wave64s.  All waves share the same 16*WM activation
//   rows; waves sit side by side along N (WAVES_N) and/or split the K-blocks
//   of a stage (WAVES_K, reduced through LDS at the end).
// * Activations are staged through LDS per stage (WAVES_K K-blocks of 128),
//   double buffered, XOR-swizzled so the MFMA operand reads are conflict
//   free.  Weights stream from HBM straight into registers with one 16-byte
//   load per lane per (16-column sub-tile, K-block) -- the packed layout puts
//   exactly the MFMA operand of each lane there -- and are dequantized in
//   registers.
// * Formats:
//     F_INT          INT4/UINT4 codes become bf16 (128 + u) with one AND-OR
//                    per two codes; the MFMA accumulates a K-block in fp32
//                    and s * (P - c * sum(a)) applies scale, zero point and
//                    the 128 offset per K-block (exact for integer codes).
//     F_MXFP4_BF16   E2M1 codes are converted with their E8M0 scale by
//                    v_cvt_scalef32_pk_bf16_fp4 (exact) into bf16 MFMA.
//     F_FP8          E4M3 x E4M3 on the 16x16x128 f8f6f4 MFMA, per-token and
//                    per-channel scales in the epilogue.
//     F_MXFP4_MXFP8  E4M3 activations x E2M1 weights on the block-scaled
//                    16x16x128 MFMA with both E8M0 scales as operands.
// * Split-K across workgroups writes fp32 partials; the last workgroup of a
//   tile (atomic ticket) sums them in split order, so results are
//   deterministic run to run, and resets its ticket.  Partial sums are never
//   rounded below fp32 (the accuracy loss through a bf16 Stream-K reduction
//   reported as issue #31 on the senn-tech.com review is the case avoided).
#include "dev_common.h"
#include "hum_internal.h"

#include <type_traits>

namespace hum {

using I0 = std::integral_constant<int, 0>;
using I1 = std::integral_constant<int, 1>;

template <int FMT>
struct FmtTraits {
  static constexpr int kAElem = (FMT == F_INT || FMT == F_MXFP4_BF16) ? 2 : 1;  // activation bytes
  static constexpr int kBWords = (FMT == F_FP8) ? 2 : 1;                         // 16-B weight words / lane / K-block
  static constexpr bool kBf16Mfma = (FMT == F_INT || FMT == F_MXFP4_BF16);
};

__device__ __forceinline__ int swz(int r, int c, int a_elem) {
  return a_elem == 2 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}

__device__ __forceinline__ bf16x8_t int_dequant(uint32_t w) {
  u32x4_t o;
  o[0] = (w & 0x000F000Fu) | 0x43004300u;
  o[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
  o[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
  o[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x8_t, o);
}

__device__ __forceinline__ bf16x8_t mx_dequant(uint32_t w, float scale) {
  bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  u32x4_t o;
  o[0] = __builtin_bit_cast(uint32_t, p0);
  o[1] = __builtin_bit_cast(uint32_t, p1);
  o[2] = __builtin_bit_cast(uint32_t, p2);
  o[3] = __builtin_bit_cast(uint32_t, p3);
  return __builtin_bit_cast(bf16x8_t, o);
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

template <int FMT, int WM, int WN, int WAVES_N, int WAVES_K, int AMODE, int EPI>
struct GemmCfg {
  using T = FmtTraits<FMT>;
  static constexpr int kTM = 16 * WM;
  static constexpr int kTNS = WN * WAVES_N;  // sub-tiles per workgroup (weight space)
  static constexpr int kRowB = 128 * T::kAElem;
  static constexpr int kCPR = kRowB / 16;
  static constexpr int kKbBytes = kTM * kRowB;
  static constexpr int kStageA = WAVES_K * kKbBytes;
  static constexpr int kStageRs = (FMT == F_INT) ? WAVES_K * kTM * 4 : 0;
  static constexpr int kStageAs = (FMT == F_MXFP4_MXFP8) ? WAVES_K * kTM * 4 : 0;
  static constexpr int kStage = kStageA + kStageRs + kStageAs;
  static constexpr int kChunks = WAVES_K * kTM * kCPR;
  static constexpr int kCPT = (kChunks + 255) / 256;
  static constexpr int kAccPerWave = WM * WN * 4 * 64;  // floats
  static constexpr int kRedBytes = (WAVES_K - 1) * WAVES_N * kAccPerWave * 4;
  static constexpr int kLds = (2 * kStage > kRedBytes) ? 2 * kStage : kRedBytes;
  static constexpr bool kSwiglu = (EPI == EPI_SWIGLU_BF16 || EPI == EPI_SWIGLU_MXFP8);
  static_assert(WAVES_N * WAVES_K == 4, "4 waves per workgroup");
  static_assert(!kSwiglu || (WN % 2 == 0), "SwiGLU needs gate/up sub-tile pairs");
  static_assert(EPI != EPI_SWIGLU_MXFP8 || (WN % 4 == 0), "MXFP8 epilogue needs 32-column blocks");
  static_assert(kLds <= 160 * 1024, "LDS budget");
};

template <int FMT, int WM, int WN, int WAVES_N, int WAVES_K, int AMODE, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmParams p) {
  using C = GemmCfg<FMT, WM, WN, WAVES_N, WAVES_K, AMODE, EPI>;
  using Tr = typename C::T;
  constexpr int kAE = Tr::kAElem;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::kLds];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WAVES_N, wk = wave / WAVES_N;
  const int c16 = lane & 15, lg = lane >> 4;

  int64_t bid = blockIdx.x;
  const int split = (int)(bid % p.split_k);
  bid /= p.split_k;
  const int tn = (int)(bid % p.n_tiles);
  const int64_t tm = bid / p.n_tiles;
  const int64_t tile_id = tm * p.n_tiles + tn;

  int expert = 0;
  if (AMODE == A_GATHER || EPI == EPI_SCATTER) {
    expert = p.block_expert[tm];
    if (expert < 0) return;  // block past the last expert segment
  }
  const int64_t row0 = tm * C::kTM;
  const uint8_t* codes = p.codes + (int64_t)expert * p.codes_per_expert;
  const uint8_t* wmeta = p.wscale + (int64_t)expert * p.scales_per_expert;
  const uint8_t* wzero = p.wzero ? p.wzero + (int64_t)expert * p.zeros_per_expert : nullptr;
  const float gs = p.gscale[expert];

  // This wave's 16-column sub-tiles (weight space) and their validity.
  int nts[WN];
  bool ntv[WN];
#pragma unroll
  for (int ns = 0; ns < WN; ++ns) {
    if (C::kSwiglu) {
      const int j = ns % (WN / 2);
      const int ntg = tn * (C::kTNS / 2) + wn * (WN / 2) + j;
      ntv[ns] = ntg * 16 < p.n;
      nts[ns] = ntg + (ns >= WN / 2 ? p.swiglu_nt_off : 0);
    } else {
      nts[ns] = tn * C::kTNS + wn * WN + ns;
      ntv[ns] = nts[ns] < p.nt_count;
    }
  }

  const int kb_begin = split * p.kb_per_split;
  int kb_end = kb_begin + p.kb_per_split;
  if (kb_end > p.kb_count) kb_end = p.kb_count;
  const int n_kb = kb_end > kb_begin ? kb_end - kb_begin : 0;
  const int n_stages = (n_kb + WAVES_K - 1) / WAVES_K;

  // ---- activation row sources of this thread's staging chunks --------------
  const uint8_t* a_row[C::kCPT];
  int ch_off[C::kCPT];  // LDS offset inside a stage
  int ch_kbl[C::kCPT];
  int ch_col[C::kCPT];
  bool ch_ok[C::kCPT];
#pragma unroll
  for (int i = 0; i < C::kCPT; ++i) {
    const int id = tid + 256 * i;
    ch_ok[i] = id < C::kChunks;
    const int kbl = id / (C::kTM * C::kCPR);
    const int rem = id % (C::kTM * C::kCPR);
    const int r = rem / C::kCPR, c = rem % C::kCPR;
    ch_kbl[i] = kbl;
    ch_col[i] = c;
    ch_off[i] = kbl * C::kKbBytes + r * C::kRowB + swz(r, c, kAE) * 16;
    const int64_t row = row0 + r;
    const uint8_t* src = nullptr;
    if (ch_ok[i]) {
      if (AMODE == A_GATHER) {
        const int32_t f = row < p.m ? p.sorted[row] : p.sentinel;
        if (f < p.sentinel) src = static_cast<const uint8_t*>(p.a) + (int64_t)(f / p.topk) * p.lda * kAE;
      } else if (row < p.m) {
        src = static_cast<const uint8_t*>(p.a) + row * p.lda * kAE;
      }
    }
    a_row[i] = src;
  }
  // MXFP8 activation scale rows (one dword = the 4 E8M0 codes of a K-block)
  const uint8_t* as_row = nullptr;
  int as_off = 0, as_kbl = 0;
  if (FMT == F_MXFP4_MXFP8 && tid < WAVES_K * C::kTM) {
    as_kbl = tid / C::kTM;
    const int r = tid % C::kTM;
    as_off = C::kStageA + C::kStageRs + (as_kbl * C::kTM + r) * 4;
    const int64_t row = row0 + r;
    if (AMODE == A_GATHER) {
      const int32_t f = row < p.m ? p.sorted[row] : p.sentinel;
      if (f < p.sentinel) as_row = static_cast<const uint8_t*>(p.a_scale) + (int64_t)(f / p.topk) * p.a_scale_ld;
    } else if (row < p.m) {
      as_row = static_cast<const uint8_t*>(p.a_scale) + row * p.a_scale_ld;
    }
  }

  u32x4_t a_reg[C::kCPT];
  uint32_t as_reg = 0x7F7F7F7Fu;
  auto load_a = [&](int st) {
#pragma unroll
    for (int i = 0; i < C::kCPT; ++i) {
      const int kb = kb_begin + st * WAVES_K + ch_kbl[i];
      u32x4_t v = {0, 0, 0, 0};
      if (a_row[i] && kb < kb_end)
        v = *reinterpret_cast<const u32x4_t*>(a_row[i] + (int64_t)kb * 128 * kAE + ch_col[i] * 16);
      a_reg[i] = v;
    }
    if (FMT == F_MXFP4_MXFP8) {
      const int kb = kb_begin + st * WAVES_K + as_kbl;
      as_reg = 0x7F7F7F7Fu;
      if (as_row && kb < kb_end) as_reg = *reinterpret_cast<const uint32_t*>(as_row + (int64_t)kb * 4);
    }
  };
  auto store_a = [&](int buf) {
    uint8_t* base = smem + buf * C::kStage;
#pragma unroll
    for (int i = 0; i < C::kCPT; ++i) {
      if (!ch_ok[i]) continue;
      *reinterpret_cast<u32x4_t*>(base + ch_off[i]) = a_reg[i];
      if (FMT == F_INT) {
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) s += bf16_bits_to_f32(a_reg[i][q] & 0xFFFF) + bf16_bits_to_f32(a_reg[i][q] >> 16);
        s = row16_sum(s);  // the 16 chunks of one row's K-block are one DPP row
        if (ch_col[i] == 0) {
          const int id = tid + 256 * i;
          const int r = (id % (C::kTM * C::kCPR)) / C::kCPR;
          reinterpret_cast<float*>(base + C::kStageA)[ch_kbl[i] * C::kTM + r] = s;
        }
      }
    }
    if (FMT == F_MXFP4_MXFP8 && tid < WAVES_K * C::kTM)
      *reinterpret_cast<uint32_t*>(base + as_off) = as_reg;
  };

  // ---- weights -------------------------------------------------------------
  u32x4_t bw[2][WN][Tr::kBWords];
  uint32_t bm[2][WN];   // meta: INT scale bits / MX scale dword
  uint32_t bz[2][WN];   // INT zero nibble
  auto load_b = [&](int st, auto set_c) {
    constexpr int set = decltype(set_c)::value;
    const int kb = kb_begin + st * WAVES_K + wk;
    const bool kok = kb < kb_end;
#pragma unroll
    for (int ns = 0; ns < WN; ++ns) {
      const bool ok = kok && ntv[ns];
      const int64_t blk = ((int64_t)nts[ns] * p.kb_count + kb) * 64 + lane;
#pragma unroll
      for (int w = 0; w < Tr::kBWords; ++w) {
        u32x4_t v = {0, 0, 0, 0};
        if (ok) v = *reinterpret_cast<const u32x4_t*>(codes + blk * (16 * Tr::kBWords) + 16 * w);
        bw[set][ns][w] = v;
      }
      if (FMT == F_INT) {
        uint32_t sbits = 0, z = 0;
        if (ok) {
          const int g = kb / p.kb_per_group;
          const int64_t gi = (int64_t)nts[ns] * p.ng + g;
          sbits = p.scale_f32 ? reinterpret_cast<const uint32_t*>(wmeta)[gi * 16 + c16]
                              : (uint32_t)reinterpret_cast<const uint16_t*>(wmeta)[gi * 16 + c16] << 16;
          if (p.has_zero) z = (uint32_t)(reinterpret_cast<const uint64_t*>(wzero)[gi] >> (4 * c16)) & 0xF;
        }
        bm[set][ns] = sbits;
        bz[set][ns] = z;
      } else if (FMT == F_MXFP4_BF16 || FMT == F_MXFP4_MXFP8) {
        uint32_t word = 0x7F7F7F7Fu;
        if (ok) word = reinterpret_cast<const uint32_t*>(wmeta)[((int64_t)nts[ns] * p.kb4 + kb / 4) * 64 + lane];
        bm[set][ns] = (word >> (8 * (kb & 3))) & 0xFF;
      }
    }
  };

  f32x4_t acc[WM][WN];
#pragma unroll
  for (int ms = 0; ms < WM; ++ms)
#pragma unroll
    for (int ns = 0; ns < WN; ++ns) acc[ms][ns] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](int st, int buf, auto set_c) {
    constexpr int set = decltype(set_c)::value;
    const int kb = kb_begin + st * WAVES_K + wk;
    if (kb >= kb_end) return;
    const uint8_t* abase = smem + buf * C::kStage + wk * C::kKbBytes;
    if constexpr (Tr::kBf16Mfma) {
      bf16x8_t deq[WN][4];
      float sc[WN], off[WN];
#pragma unroll
      for (int ns = 0; ns < WN; ++ns) {
        if (FMT == F_INT) {
#pragma unroll
          for (int s = 0; s < 4; ++s) deq[ns][s] = int_dequant(bw[set][ns][0][s]);
          sc[ns] = __uint_as_float(bm[set][ns]);
          off[ns] = (float)(p.int_offset + (int)bz[set][ns]);
        } else {
          const float fs = e8m0_to_f32(bm[set][ns]);
#pragma unroll
          for (int s = 0; s < 4; ++s) deq[ns][s] = mx_dequant(bw[set][ns][0][s], fs);
        }
      }
#pragma unroll
      for (int ms = 0; ms < WM; ++ms) {
        const int r = ms * 16 + c16;
        bf16x8_t af[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
          af[s] = *reinterpret_cast<const bf16x8_t*>(abase + r * C::kRowB + (((4 * lg + s) ^ c16) * 16));
        if constexpr (FMT == F_INT) {
          const f32x4_t rs = *reinterpret_cast<const f32x4_t*>(
              smem + buf * C::kStage + C::kStageA + (wk * C::kTM + ms * 16 + 4 * lg) * 4);
#pragma unroll
          for (int ns = 0; ns < WN; ++ns) {
            f32x4_t t = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], deq[ns][s], t, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[ms][ns][i] = __builtin_fmaf(sc[ns], __builtin_fmaf(-off[ns], rs[i], t[i]), acc[ms][ns][i]);
          }
        } else {
#pragma unroll
          for (int ns = 0; ns < WN; ++ns)
#pragma unroll
            for (int s = 0; s < 4; ++s)
              acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], deq[ns][s], acc[ms][ns], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int ms = 0; ms < WM; ++ms) {
        const int r = ms * 16 + c16;
        const int sw = (r >> 1) & 7;
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(abase + r * C::kRowB + ((lg ^ sw) * 16));
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(abase + r * C::kRowB + (((4 + lg) ^ sw) * 16));
        i32x8_t a8;
        a8[0] = lo[0]; a8[1] = lo[1]; a8[2] = lo[2]; a8[3] = lo[3];
        a8[4] = hi[0]; a8[5] = hi[1]; a8[6] = hi[2]; a8[7] = hi[3];
        int sa = 127;
        if (FMT == F_MXFP4_MXFP8)
          sa = (int)((reinterpret_cast<const uint32_t*>(smem + buf * C::kStage + C::kStageA + C::kStageRs)
                          [wk * C::kTM + r] >> (8 * lg)) & 0xFF);
#pragma unroll
        for (int ns = 0; ns < WN; ++ns) {
          i32x8_t b8;
          if (FMT == F_FP8) {
            b8[0] = bw[set][ns][0][0]; b8[1] = bw[set][ns][0][1]; b8[2] = bw[set][ns][0][2]; b8[3] = bw[set][ns][0][3];
            b8[4] = bw[set][ns][Tr::kBWords - 1][0]; b8[5] = bw[set][ns][Tr::kBWords - 1][1];
            b8[6] = bw[set][ns][Tr::kBWords - 1][2]; b8[7] = bw[set][ns][Tr::kBWords - 1][3];
            acc[ms][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[ms][ns], 0, 0, 0, 127, 0, 127);
          } else {
            b8[0] = bw[set][ns][0][0]; b8[1] = bw[set][ns][0][1]; b8[2] = bw[set][ns][0][2]; b8[3] = bw[set][ns][0][3];
            b8[4] = 0; b8[5] = 0; b8[6] = 0; b8[7] = 0;
            acc[ms][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[ms][ns], 0, 4, 0, sa, 0,
                                                                           (int)bm[set][ns]);
          }
        }
      }
    }
  };

  // ---- main loop: A double-buffered in LDS, B double-buffered in registers --
  if (n_stages > 0) {
    load_a(0);
    load_b(0, I0{});
    store_a(0);
    __syncthreads();
    for (int st = 0; st < n_stages; st += 2) {
      const bool n1 = st + 1 < n_stages;
      if (n1) {
        load_a(st + 1);
        load_b(st + 1, I1{});
      }
      compute(st, 0, I0{});
      if (n1) store_a(1);
      __syncthreads();
      if (!n1) break;
      const bool n2 = st + 2 < n_stages;
      if (n2) {
        load_a(st + 2);
        load_b(st + 2, I0{});
      }
      compute(st + 1, 1, I1{});
      if (n2) store_a(0);
      __syncthreads();
    }
  }

  // ---- in-workgroup split-K: waves wk > 0 hand their sums to wk == 0 -------
  if constexpr (WAVES_K > 1) {
    float* red = reinterpret_cast<float*>(smem);
    if (wk > 0) {
      float* dst = red + ((wk - 1) * WAVES_N + wn) * C::kAccPerWave;
#pragma unroll
      for (int ms = 0; ms < WM; ++ms)
#pragma unroll
        for (int ns = 0; ns < WN; ++ns)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[((ms * WN + ns) * 4 + i) * 64 + lane] = acc[ms][ns][i];
    }
    __syncthreads();
    if (wk == 0) {
      for (int q = 1; q < WAVES_K; ++q) {
        const float* src = red + ((q - 1) * WAVES_N + wn) * C::kAccPerWave;
#pragma unroll
        for (int ms = 0; ms < WM; ++ms)
#pragma unroll
          for (int ns = 0; ns < WN; ++ns)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[ms][ns][i] += src[((ms * WN + ns) * 4 + i) * 64 + lane];
      }
    }
  }

  // ---- cross-workgroup split-K: fp32 partials, last arrival reduces ---------
  if (p.split_k > 1) {
    float* part = p.partials + (tile_id * p.split_k * WAVES_N) * (int64_t)C::kAccPerWave;
    if (wk == 0) {
      float* dst = part + ((int64_t)split * WAVES_N + wn) * C::kAccPerWave;
#pragma unroll
      for (int ms = 0; ms < WM; ++ms)
#pragma unroll
        for (int ns = 0; ns < WN; ++ns)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[((ms * WN + ns) * 4 + i) * 64 + lane] = acc[ms][ns][i];
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int prev = atomicAdd(&p.counters[tile_id], 1);
      s_last = (prev == p.split_k - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (wk == 0) {
#pragma unroll
      for (int ms = 0; ms < WM; ++ms)
#pragma unroll
        for (int ns = 0; ns < WN; ++ns) acc[ms][ns] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      for (int q = 0; q < p.split_k; ++q) {
        const float* src = part + ((int64_t)q * WAVES_N + wn) * C::kAccPerWave;
#pragma unroll
        for (int ms = 0; ms < WM; ++ms)
#pragma unroll
          for (int ns = 0; ns < WN; ++ns)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[ms][ns][i] += __builtin_nontemporal_load(&src[((ms * WN + ns) * 4 + i) * 64 + lane]);
      }
    }
    if (tid == 0) p.counters[tile_id] = 0;  // ready for the next call
  }

  if (wk != 0) return;

  // ---- epilogues -------------------------------------------------------------
  if constexpr (EPI == EPI_BF16 || EPI == EPI_SCATTER) {
    uint16_t* out = static_cast<uint16_t*>(p.out);
#pragma unroll
    for (int ns = 0; ns < WN; ++ns) {
      const int64_t col = (int64_t)nts[ns] * 16 + c16;
      if (col >= p.n) continue;
      float cs = gs;
      if (FMT == F_FP8) cs *= reinterpret_cast<const float*>(wmeta)[col];
      const float bias = (EPI == EPI_BF16 && p.bias) ? bf16_bits_to_f32(p.bias[col]) : 0.0f;
#pragma unroll
      for (int ms = 0; ms < WM; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t row = row0 + ms * 16 + 4 * lg + i;
          if (row >= p.m) continue;
          float v = acc[ms][ns][i] * cs;
          if (FMT == F_FP8) v *= reinterpret_cast<const float*>(p.a_scale)[row];
          v += bias;
          if (EPI == EPI_SCATTER) {
            const int32_t f = p.sorted[row];
            if (f >= p.sentinel) continue;
            out[(int64_t)f * p.ldo + col] = (uint16_t)f32_to_bf16_bits(v);
          } else {
            out[row * p.ldo + col] = (uint16_t)f32_to_bf16_bits(v);
          }
        }
    }
  } else if constexpr (EPI == EPI_SWIGLU_BF16) {
    uint16_t* out = static_cast<uint16_t*>(p.out);
#pragma unroll
    for (int j = 0; j < WN / 2; ++j) {
      const int64_t col = (int64_t)nts[j] * 16 + c16;
      if (col >= p.n) continue;
#pragma unroll
      for (int ms = 0; ms < WM; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t row = row0 + ms * 16 + 4 * lg + i;
          const float g = acc[ms][j][i] * gs, u = acc[ms][j + WN / 2][i] * gs;
          out[row * p.ldo + col] = (uint16_t)f32_to_bf16_bits(silu_f32(g) * u);
        }
    }
  } else {  // EPI_SWIGLU_MXFP8: 32-column blocks = gate sub-tile pairs
    uint8_t* outq = static_cast<uint8_t*>(p.out);
    uint8_t* outs = static_cast<uint8_t*>(p.out_scale);
#pragma unroll
    for (int jj = 0; jj < WN / 4; ++jj) {
      const int j0 = 2 * jj, j1 = 2 * jj + 1;
      const int64_t col0 = (int64_t)nts[j0] * 16 + c16, col1 = (int64_t)nts[j1] * 16 + c16;
      const bool ok = nts[j0] * 16 < p.n;  // whole 32-block valid (I % 32 == 0)
#pragma unroll
      for (int ms = 0; ms < WM; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t row = row0 + ms * 16 + 4 * lg + i;
          const float a0 = silu_f32(acc[ms][j0][i] * gs) * (acc[ms][j0 + WN / 2][i] * gs);
          const float a1 = silu_f32(acc[ms][j1][i] * gs) * (acc[ms][j1 + WN / 2][i] * gs);
          const float amax = row16_max(__builtin_fmaxf(__builtin_fabsf(a0), __builtin_fabsf(a1)));
          const int e = mx_scale_code(amax);
          const float inv = mx_inv_scale(e);
          const uint32_t q = f32x2_to_e4m3x2(a0 * inv, a1 * inv);
          if (ok) {
            outq[row * p.ldo + col0] = (uint8_t)(q & 0xFF);
            outq[row * p.ldo + col1] = (uint8_t)(q >> 8);
            if (c16 == 0) outs[row * (p.ldo / 32) + col0 / 32] = (uint8_t)e;
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Instances.  The selector only returns keys listed here.

typedef void (*gemm_fn)(const GemmParams);

struct Instance {
  KernelKey key;
  gemm_fn fn;
};

#define HUM_INST(F, WM, WN, WVN, WVK, AM, EP) \
  {{F, WM, WN, WVN, WVK, AM, EP}, gemm_kernel<F, WM, WN, WVN, WVK, AM, EP>}

#define HUM_DENSE_SET(F)                                 \
  HUM_INST(F, 1, 1, 1, 4, A_DIRECT, EPI_BF16),           \
  HUM_INST(F, 1, 2, 2, 2, A_DIRECT, EPI_BF16),           \
  HUM_INST(F, 1, 4, 4, 1, A_DIRECT, EPI_BF16),           \
  HUM_INST(F, 2, 2, 2, 2, A_DIRECT, EPI_BF16),           \
  HUM_INST(F, 4, 2, 2, 2, A_DIRECT, EPI_BF16),           \
  HUM_INST(F, 4, 4, 4, 1, A_DIRECT, EPI_BF16),           \
  HUM_INST(F, 8, 4, 4, 1, A_DIRECT, EPI_BF16)

#define HUM_MOE_SET(F, EPI_UP)                           \
  HUM_INST(F, 1, 4, 1, 4, A_GATHER, EPI_UP),             \
  HUM_INST(F, 1, 4, 2, 2, A_GATHER, EPI_UP),             \
  HUM_INST(F, 2, 4, 2, 2, A_GATHER, EPI_UP),             \
  HUM_INST(F, 4, 4, 4, 1, A_GATHER, EPI_UP),             \
  HUM_INST(F, 8, 4, 4, 1, A_GATHER, EPI_UP),             \
  HUM_INST(F, 1, 4, 1, 4, A_DIRECT, EPI_SCATTER),        \
  HUM_INST(F, 1, 4, 2, 2, A_DIRECT, EPI_SCATTER),        \
  HUM_INST(F, 2, 4, 2, 2, A_DIRECT, EPI_SCATTER),        \
  HUM_INST(F, 4, 4, 4, 1, A_DIRECT, EPI_SCATTER),        \
  HUM_INST(F, 8, 4, 4, 1, A_DIRECT, EPI_SCATTER)

static const Instance kInstances[] = {
    HUM_DENSE_SET(F_INT),
    HUM_DENSE_SET(F_FP8),
    HUM_DENSE_SET(F_MXFP4_BF16),
    HUM_MOE_SET(F_MXFP4_BF16, EPI_SWIGLU_BF16),
    HUM_MOE_SET(F_MXFP4_MXFP8, EPI_SWIGLU_MXFP8),
};

static const Instance* find_instance(const KernelKey& k) {
  for (const Instance& in : kInstances) {
    const KernelKey& q = in.key;
    if (q.fmt == k.fmt && q.wm == k.wm && q.wn == k.wn && q.waves_n == k.waves_n && q.waves_k == k.waves_k &&
        q.amode == k.amode && q.epi == k.epi)
      return &in;
  }
  return nullptr;
}

bool gemm_instance_exists(const KernelKey& key) { return find_instance(key) != nullptr; }

hum_status launch_gemm(const KernelKey& key, const GemmParams& p, int64_t m_tiles, void* stream) {
  const Instance* in = find_instance(key);
  if (!in)
    return set_error(HUM_ERR_UNSUPPORTED, "no GEMM instance fmt=%d wm=%d wn=%d waves_n=%d waves_k=%d amode=%d epi=%d",
                     key.fmt, key.wm, key.wn, key.waves_n, key.waves_k, key.amode, key.epi);
  const int64_t grid = m_tiles * (int64_t)p.n_tiles * p.split_k;
  if (grid <= 0) return HUM_OK;
  if (grid > 0x7FFFFFFF) return set_error(HUM_ERR_UNSUPPORTED, "grid too large");
  hipLaunchKernelGGL(in->fn, dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream), p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "gemm launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

}  // namespace hum
