// Quantized GEMM for gfx950: dense layers and grouped (MoE) expert layers.
//
// What is computed is the WnA16 / W8A8 / W4A8 GEMM of "Announcing Humming:
// Fast, Flexible Kernels for Quantized Inference" (sections "WnA16" and
// "W8A8 / W4A8 / W4A4"): dequantization and scaling fused into the GEMM
// (section "Shared CUDA components"), a task mapping per GEMM type for dense
// and MoE work, scale / bias epilogues.  The design is gfx950's own.
//
// Two kernel families share the fragment, MFMA and epilogue code below:
//
// * stream_kernel (decode, one 16-row tile): KW wave64s of a workgroup split
//   the K range of the same WN 16-column sub-tiles.  Weights stream from HBM
//   straight into a register ring PF K-blocks deep (one 16-byte load per
//   lane per sub-tile and K-block -- the packed layout puts exactly each
//   lane's MFMA operand there); the activation rows and the weight metadata
//   of the K range are staged in LDS once.  No barrier until the final
//   in-workgroup reduction through LDS.
// * tile_kernel (prefill): 4 waves side by side along N share a 16*WM-row
//   activation tile.  Each K-block's activation tile (XOR swizzled so the
//   operand reads are conflict free) and metadata are copied global -> LDS
//   by buffer-load-to-LDS DMA, one or two K-blocks ahead; each wave loads
//   its own weight fragments straight into registers and dequantizes them
//   there.  Workgroups are ordered so that the tiles one XCD runs at a time
//   share activation rows and weight columns in its L2.
//
// Formats:
//   F_INT          INT4/UINT4 -> bf16 (128 + u) with one AND-OR per two
//                  codes (F_INT3 / F_INT2 / F_INT1: b-bit codes from bit
//                  planes, one or two AND-ORs per two codes); a K-block accumulates in fp32 and
//                  s * (P - (128 + z) * sum(a)) applies scale, zero point and
//                  the offset (exact for integer codes).
//   F_MXFP4_BF16   E2M1 with its E8M0 scale -> bf16 through
//                  v_cvt_scalef32_pk_bf16_fp4 (exact), bf16 MFMA.
//   F_FP8          E4M3 x E4M3 on the 16x16x128 f8f6f4 MFMA; per-token and
//                  per-channel scales in the epilogue.
//   F_MXFP4_MXFP8  E4M3 activations x E2M1 weights on the block-scaled
//                  16x16x128 MFMA, both E8M0 scales as operands.
//   F_MXFP4_MXFP4  E2M1 activations x E2M1 weights (W4A4) on the same
//                  MFMA; tile kernels (at decode sizes W4A4 runs on the
//                  F_MXFP4_MXFP8 decode kernel, its MXFP4 activations handed
//                  over as the E4M3 bytes of the same values).
//   F_FP8_BF16     E4M3 weights x bf16 activations (W8A16): the hardware
//                  FP8 -> bf16 conversion (exact), bf16 MFMA, per-channel
//                  scales in the epilogue.
//   F_INT8_BF16    INT8 weights x bf16 activations (W8A16): bytes widened
//                  through f32 (exact), the FP8 path's layout and epilogue.
//   F_NVFP4_BF16   NVFP4: E2M1 -> f32, times its E4M3 scale per 16 (exact: at
//                  most 6 significant bits) -> bf16.
//   F_MXFP6_BF16 / F_MXBF6_BF16  MXFP6 (E2M3 / E3M2 with an E8M0 scale per
//                  32): the 32-wide hardware FP6 -> bf16 conversion, bf16 MFMA.
//   F_MXINT4_BF16  MXINT4: INT4 with an E8M0 scale per 32 -> f32 -> bf16
//                  (exact), the MX path's scale staging.
//   F_FP8_BLOCK    block-scaled FP8: E4M3 x E4M3 on the same MFMA one
//                  K-block (128) at a time, each K-block's result scaled by
//                  the row's group scale times the 128 x 128 weight-block
//                  scale (acc += sa * sw * P); tile kernels, and the dense
//                  decode kernel, which quantizes each row's K-blocks itself.
//
// Split-K across workgroups writes fp32 partials; a separate reduce kernel
// sums them in split order (deterministic) and applies the epilogue.
// Partial sums are never rounded below fp32 (the accuracy loss through a bf16
// Stream-K reduction, issue #31 in the senn-tech.com review, is what this
// avoids).
#pragma once

#include "dev_common.h"
#include "hum_internal.h"

#include <type_traits>

namespace hum {

template <int FMT>
struct Tr {
  static constexpr int kAElem = fmt_bf16_act(FMT) ? 2 : 1;  // activation bytes (FP4: 1/2)
  static constexpr bool kA4 = (FMT == F_MXFP4_MXFP4);                           // 4-bit activations
  static constexpr int kARowB = kA4 ? 64 : 128 * kAElem;                        // activation bytes per row per K-block
  static constexpr int kBWords =
      (FMT == F_FP8 || FMT == F_FP8_BLOCK || fmt_w8_bf16(FMT)) ? 2 : 1;  // 16-B words / lane / K-block
  static constexpr bool kBf16 = fmt_bf16_act(FMT);
  // integer family: bits per code; code bytes per lane per K-block (b-bit
  // integers: 4b, else 16 per 16-byte word)
  static constexpr int kIntBits = fmt_int_bits(FMT);
  static constexpr int kCodeB = fmt_int(FMT) ? 4 * kIntBits : (fmt_fp6(FMT) ? 24 : 16 * kBWords);
  // MX / NVFP4 weight scales: a metadata row (a dword per lane) covers
  // 1 << kMetaRowShift K-blocks (E8M0 per 32: 4; NVFP4's two E4M3 per 32: 2)
  static constexpr int kMetaRowShift = FMT == F_NVFP4_BF16 ? 1 : 2;
  // bytes of an activation row of `ld` elements
  static __device__ __forceinline__ int64_t row_bytes(int64_t ld) { return kA4 ? ld / 2 : ld * kAElem; }
};

// ---------------------------------------------------------------------------
// Weight fragments

// A lane's code words of one K-block: 16-byte words, or for b-bit integers
// (b < 4) b dwords.
template <int B>
struct CodeWord { using type = u32x4_t; };
template <> struct CodeWord<24> { using type = u32x6_t; };
template <> struct CodeWord<12> { using type = u32x3_t; };
template <> struct CodeWord<8> { using type = u32x2_t; };
template <> struct CodeWord<4> { using type = u32x1_t; };

template <int FMT>
using CodeW = typename CodeWord<(Tr<FMT>::kCodeB < 16 || Tr<FMT>::kCodeB == 24) ? Tr<FMT>::kCodeB : 16>::type;

// One buffer load of a lane's code word (16-byte words: one of them).
template <int FMT>
__device__ __forceinline__ CodeW<FMT> load_code_word(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  constexpr int B = Tr<FMT>::kCodeB;
  if constexpr (B == 4) {
    CodeW<FMT> w;
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    return w;
  } else if constexpr (B == 8) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  } else if constexpr (B == 12) {
    return __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
  } else if constexpr (B == 24) {
    const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    const u32x2_t b = __builtin_amdgcn_raw_buffer_load_b64(r, off + 16, 0, 0);
    return CodeW<FMT>{a[0], a[1], a[2], a[3], b[0], b[1]};
  } else {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  }
}

template <int FMT>
struct BFrag {
  CodeW<FMT> w[Tr<FMT>::kBWords];
  // raw metadata words as loaded (decoded where the fragment is used, so
  // that no arithmetic waits on a load where it is issued)
  uint32_t meta;  // INT: dword holding the column's scale; MX: E8M0 codes of 4 K-blocks
  uint32_t zero;  // INT: dword holding the column's zero-point nibble
};

struct WPtrs {
  const uint8_t* codes;
  const uint8_t* meta;
  const uint8_t* zero;
};

// Buffer resources over the weight stripe of one 16-column sub-tile (its
// codes and metadata for the whole K).  A fragment outside the stripe -- a
// K-block past the end of the wave's range, or a sub-tile past N (range 0)
// -- is read at an offset beyond the range: the hardware returns zeros and
// touches no memory.  So every weight load is unconditional (a load inside a
// branch makes the compiler wait for all outstanding loads where the branch
// rejoins, which would serialize the prefetch ring) and costs nothing when
// unused.
struct WStripe {
  __amdgpu_buffer_rsrc_t codes, meta, zero;
};

constexpr uint32_t kOob = 0x80000000u;  // beyond every stripe (stripes are < 2 GiB)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// The same descriptor as four words, for LDS DMA issued from inline assembly.
__device__ __forceinline__ u32x4_t rsrc_words(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, (uint32_t)bytes, 0x00020000u};
}

// LDS DMA (buffer_load ... lds): lane l's 16 (4) bytes at byte offset voff of
// the buffer land at lds + 16 l (4 l).  Issued from inline assembly so that
// the compiler keeps no count of it and adds no waits of its own for the
// LDS it writes: the kernel waits itself (s_waitcnt vmcnt), knowing which
// copies it needs.  The instruction has no register result, so nothing of
// the asm statement is left in flight but the copy itself.
__device__ __forceinline__ uint32_t lds_addr(const void* lds) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
}
__device__ __forceinline__ void dma_b128(u32x4_t r, const void* lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_addr(lds)), "v"(voff), "s"(r) : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(u32x4_t r, const void* lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds_addr(lds)), "v"(voff), "s"(r) : "memory", "m0");
}

template <int FMT>
__device__ __forceinline__ WStripe make_stripe(const GemmParams& p, const WPtrs& w, int nt, bool valid) {
  constexpr int kCB = Tr<FMT>::kCodeB;  // code bytes per lane per K-block
  const int64_t ntc = valid ? nt : 0;
  WStripe s;
  const int64_t cb = (int64_t)p.kb_count * 64 * kCB;
  s.codes = make_rsrc(w.codes + ntc * cb, valid ? cb : 0);
  s.meta = s.codes;
  s.zero = s.codes;
  if (fmt_int(FMT)) {
    const int64_t sb = (int64_t)p.ng * 16 * (p.scale_f32 ? 4 : 2);
    s.meta = make_rsrc(w.meta + ntc * sb, valid ? sb : 0);
    const int64_t zb = (int64_t)p.ng * 8;
    s.zero = make_rsrc(w.zero + ntc * zb, (valid && p.has_zero) ? zb : 0);
  } else if (fmt_mx_meta(FMT)) {
    const int64_t sb = (int64_t)p.kb4 * 256;
    s.meta = make_rsrc(w.meta + ntc * sb, valid ? sb : 0);
  }
  return s;
}

// Loads of one weight fragment (K-block kb of the stripe; zeros when !ok).
// META = false loads the codes only (the caller holds the metadata).
template <int FMT, bool META = true>
__device__ __forceinline__ BFrag<FMT> load_b(const GemmParams& p, const WStripe& s, bool ok, int kb, int lane) {
  constexpr int kCB = Tr<FMT>::kCodeB;
  BFrag<FMT> f;
  const uint32_t co = ok ? (uint32_t)(kb * 64 + lane) * kCB : kOob;
#pragma unroll
  for (int i = 0; i < Tr<FMT>::kBWords; ++i) f.w[i] = load_code_word<FMT>(s.codes, co + 16 * i);
  f.meta = 0;
  f.zero = 0;
  if (META && fmt_int(FMT)) {
    const int c16 = lane & 15;
    // floor(kb / kb_per_group), exact in fp32: kb < 2^14, and the quotient
    // of (kb + 1/2) sits at least 1/(2 kb_per_group) from an integer
    const int gi = (int)(((float)kb + 0.5f) * p.inv_kbg);
    // bf16 scales: the dword holding the pair of column c16; f32: its dword
    // (arithmetic rather than a select on the uniform format flag, which
    // the compiler would turn into a branch around the load)
    const int sf = p.scale_f32;
    const uint32_t so = ok ? (uint32_t)(gi * 16 + (c16 & (14 | sf))) << (1 + sf) : kOob;
    f.meta = __builtin_amdgcn_raw_buffer_load_b32(s.meta, so, 0, 0);
    const uint32_t zo = ok ? (uint32_t)gi * 8 + ((c16 >> 3) << 2) : kOob;
    f.zero = __builtin_amdgcn_raw_buffer_load_b32(s.zero, zo, 0, 0);
  } else if (META && (fmt_mx_meta(FMT))) {
    const uint32_t mo = ok ? (uint32_t)((kb >> Tr<FMT>::kMetaRowShift) * 64 + lane) * 4 : kOob;
    f.meta = __builtin_amdgcn_raw_buffer_load_b32(s.meta, mo, 0, 0);
  }
  return f;
}

// Decoders of a fragment's metadata words.  The INT scale of column c16 is
// (raw << sh) & mk: f32 scales sh = 0, mk = ~0; bf16 pairs take the low
// half (sh = 16) for even columns and the high half (mk = 0xFFFF0000) for
// odd ones.
struct IntScaleSel {
  uint32_t sh, mk;
};
__device__ __forceinline__ IntScaleSel int_scale_sel(const GemmParams& p, int c16) {
  const bool half = p.scale_f32 == 0;
  return IntScaleSel{(half && !(c16 & 1)) ? 16u : 0u, (half && (c16 & 1)) ? 0xFFFF0000u : 0xFFFFFFFFu};
}
__device__ __forceinline__ float frag_int_scale(uint32_t raw, const IntScaleSel& sel) {
  return __uint_as_float((raw << sel.sh) & sel.mk);
}
__device__ __forceinline__ int frag_int_zero(uint32_t raw, int c16) { return (int)((raw >> (4 * (c16 & 7))) & 0xF); }
__device__ __forceinline__ uint32_t frag_mx_code(uint32_t raw, int kb) { return (raw >> (8 * (kb & 3))) & 0xFF; }

// (x & mask) | magic in one instruction.  gfx9 encodes no literal in the
// three-operand form, so with the constants in sight the compiler would
// split it into two literal-carrying ones.  The empty asm statements (they
// emit nothing) hide the constants: the mask then rides in an SGPR and the
// magic in a VGPR, and the operation stays ordinary compiler-scheduled code,
// whose hazards against matrix instructions in flight the compiler tracks
// (a VALU instruction written in asm is outside that tracking).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
  asm("" : "+s"(mask));
  asm("" : "+v"(magic));
  return (x & mask) | magic;
}

__device__ __forceinline__ bf16x8_t int_dequant(uint32_t w) {
  const uint32_t m = 0x000F000Fu, g = 0x43004300u;
  u32x4_t o;
  o[0] = and_or(w, m, g);
  o[1] = and_or(w >> 4, m, g);
  o[2] = and_or(w >> 8, m, g);
  o[3] = and_or(w >> 12, m, g);
  return __builtin_bit_cast(bf16x8_t, o);
}

// bf16 operand (128 + u pairs) of 8-k step s of a b-bit integer fragment:
// the lane's code words of one K-block in the packed bit-plane order (4-bit:
// step s in dword s; 2-bit plane: step s in dword s / 2, byte pair s & 1;
// 1-bit plane: the last dword, nibble pair s).  s is a constant after
// unrolling.
template <int BITS, typename W>
__device__ __forceinline__ bf16x8_t int_dequant_step(const W& w, int s) {
  if constexpr (BITS == 4) {
    return int_dequant(w[s]);
  } else {
    const uint32_t g = 0x43004300u;
    u32x4_t o;
    if constexpr (BITS == 1) {
      const uint32_t x = w[0] >> (4 * s);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = and_or(x >> i, 0x00010001u, g);
    } else {
      const uint32_t x = w[s >> 1] >> (8 * (s & 1));
      if constexpr (BITS == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = and_or(x >> (2 * i), 0x00030003u, g);
      } else {
        // bit 2 of each code from the 1-bit plane, moved to bit 2 of its half
        const uint32_t z = (w[2] >> (4 * s)) << 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = and_or(z >> i, 0x00040004u, and_or(x >> (2 * i), 0x00030003u, g));
      }
    }
    return __builtin_bit_cast(bf16x8_t, o);
  }
}

__device__ __forceinline__ bf16x8_t mx_dequant(uint32_t w, float scale) {
  u32x4_t o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return __builtin_bit_cast(bf16x8_t, o);
}

// A finite E4M3 code (OCP FP8: bias 7, subnormal quantum 2^-9) as f32.
__device__ __forceinline__ float e4m3_scale_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -mag : mag;
}

// Byte i of w as a signed integer, in f32.
__device__ __forceinline__ float i8_to_f32(uint32_t w, int i) { return (float)(int)(int8_t)(w >> (8 * i)); }
// bf16 bits of lo in the low half, of hi in the high half, by truncation.
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Eight E2M1 codes (low nibble first) times an E4M3 group scale -> bf16.
// The hardware's scaled FP4 conversion applies only a power-of-two scale, so
// the codes are widened to f32 unscaled and multiplied by the full scale:
// exact (at most 6 significant bits), hence also exact when packed to bf16
// by taking each f32's upper half.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
__device__ __forceinline__ bf16x8_t nv_dequant(uint32_t w, float scale) {
  const f32x2_t r0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const f32x2_t r1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const f32x2_t r2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const f32x2_t r3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  u32x4_t o;
  o[0] = pack_hi16(r0[0] * scale, r0[1] * scale);
  o[1] = pack_hi16(r1[0] * scale, r1[1] * scale);
  o[2] = pack_hi16(r2[0] * scale, r2[1] * scale);
  o[3] = pack_hi16(r3[0] * scale, r3[1] * scale);
  return __builtin_bit_cast(bf16x8_t, o);
}

// bf16 B operand of the 4 k-steps of a K-block.
template <int FMT>
__device__ __forceinline__ void dequant_b(const BFrag<FMT>& f, uint32_t meta, int kb, bf16x8_t (&d)[4]) {
  if constexpr (fmt_int(FMT)) {
#pragma unroll
    for (int s = 0; s < 4; ++s) d[s] = int_dequant_step<Tr<FMT>::kIntBits>(f.w[0], s);
  } else if constexpr (FMT == F_FP8_BF16) {
    // E4M3 -> bf16 is exact (3 mantissa bits, exponents within bf16's
    // range): the hardware conversion with a unit scale, two codes per
    // instruction; k-step s takes bytes 8s .. 8s+7 of the lane's 32
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t w0 = f.w[s >> 1][2 * (s & 1)], w1 = f.w[s >> 1][2 * (s & 1) + 1];
      u32x4_t o;
      o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
      o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
      o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
      o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
      d[s] = __builtin_bit_cast(bf16x8_t, o);
    }
  } else if constexpr (fmt_fp6(FMT)) {
    // MXFP6: the lane's 32 codes of the K-block (a 6-bit stream) through the
    // hardware's 32-wide FP6 -> bf16 conversion with the E8M0 scale (exact:
    // at most 4 significant bits); element j of k-step s is bf16 8 s + j.
    // (The result is taken as a whole: per-element extraction from the
    // 32-wide vector is avoided.)
    typedef int i32x6_t __attribute__((ext_vector_type(6)));
    typedef __bf16 bf16x32_t __attribute__((ext_vector_type(32)));
    const float fs = e8m0_to_f32(frag_mx_code(meta, kb));
    const i32x6_t x = __builtin_bit_cast(i32x6_t, f.w[0]);
    bf16x32_t r;
    if constexpr (FMT == F_MXFP6_BF16)
      r = __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(x, fs);
    else
      r = __builtin_amdgcn_cvt_scalef32_pk32_bf16_bf6(x, fs);
    struct Steps { bf16x8_t s[4]; };
    const Steps st = __builtin_bit_cast(Steps, r);
#pragma unroll
    for (int s = 0; s < 4; ++s) d[s] = st.s[s];
  } else if constexpr (FMT == F_MXINT4_BF16) {
    // MXINT4: the integer path's nibble order (k-step s in dword s, element
    // j at bit (j & 1) * 16 + (j >> 1) * 4) holding q + 8; (u - 8) * 2^E is
    // one exact FMA in f32, packed to bf16 by its upper half (at most 4
    // significant bits)
    const float fs = e8m0_to_f32(frag_mx_code(meta, kb));
    const float off = -8.0f * fs;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t w = f.w[0][s];
      u32x4_t o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = __builtin_fmaf((float)((w >> (4 * i)) & 15u), fs, off);
        const float hi = __builtin_fmaf((float)((w >> (16 + 4 * i)) & 15u), fs, off);
        o[i] = pack_hi16(lo, hi);
      }
      d[s] = __builtin_bit_cast(bf16x8_t, o);
    }
  } else if constexpr (FMT == F_NVFP4_BF16) {
    // k-steps 2h and 2h + 1 (k = 32 lg + 16 h + [0, 16)) share the E4M3
    // scale in byte 2 (kb & 1) + h of the lane's word
    const uint32_t half = meta >> (16 * (kb & 1));
    const float f0 = e4m3_scale_to_f32(half & 0xFF), f1 = e4m3_scale_to_f32((half >> 8) & 0xFF);
    d[0] = nv_dequant(f.w[0][0], f0);
    d[1] = nv_dequant(f.w[0][1], f0);
    d[2] = nv_dequant(f.w[0][2], f1);
    d[3] = nv_dequant(f.w[0][3], f1);
  } else if constexpr (FMT == F_INT8_BF16) {
    // INT8 -> bf16 is exact (|q| <= 128): each byte sign-extended to f32,
    // and two f32 packed by their upper halves (whose lower halves are zero
    // for integers this small); same byte order as the FP8 branch
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t w0 = f.w[s >> 1][2 * (s & 1)], w1 = f.w[s >> 1][2 * (s & 1) + 1];
      u32x4_t o;
      o[0] = pack_hi16(i8_to_f32(w0, 0), i8_to_f32(w0, 1));
      o[1] = pack_hi16(i8_to_f32(w0, 2), i8_to_f32(w0, 3));
      o[2] = pack_hi16(i8_to_f32(w1, 0), i8_to_f32(w1, 1));
      o[3] = pack_hi16(i8_to_f32(w1, 2), i8_to_f32(w1, 3));
      d[s] = __builtin_bit_cast(bf16x8_t, o);
    }
  } else {
    const float fs = e8m0_to_f32(frag_mx_code(meta, kb));
#pragma unroll
    for (int s = 0; s < 4; ++s) d[s] = mx_dequant(f.w[0][s], fs);
  }
}

__device__ __forceinline__ f32x4_t mfma_bf16_kblock(const bf16x8_t (&a)[4], const bf16x8_t (&b)[4], f32x4_t c) {
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], b[s], c, 0, 0, 0);
  return c;
}

template <int FMT>
__device__ __forceinline__ f32x4_t mfma_f8_kblock(const i32x8_t& a8, int sa, const BFrag<FMT>& f, uint32_t meta, int kb,
                                                  f32x4_t c) {
  i32x8_t b8;
  b8[0] = f.w[0][0]; b8[1] = f.w[0][1]; b8[2] = f.w[0][2]; b8[3] = f.w[0][3];
  if (FMT == F_FP8 || FMT == F_FP8_BLOCK) {
    b8[4] = f.w[Tr<FMT>::kBWords - 1][0]; b8[5] = f.w[Tr<FMT>::kBWords - 1][1];
    b8[6] = f.w[Tr<FMT>::kBWords - 1][2]; b8[7] = f.w[Tr<FMT>::kBWords - 1][3];
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 0, 0, 0, 127, 0, 127);
  } else {
    b8[4] = 0; b8[5] = 0; b8[6] = 0; b8[7] = 0;
    // A format: E4M3 (0) or E2M1 (4, only the low 4 dwords of a8 are read)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, FMT == F_MXFP4_MXFP4 ? 4 : 0, 4, 0, sa, 0,
                                                            (int)frag_mx_code(meta, kb));
  }
}

// ---------------------------------------------------------------------------
// Epilogue pieces

// silu(g) = g / (1 + e^-g), with e^-g = 2^(-g log2 e) and the reciprocal on
// the hardware's 2^x and 1/x instructions (about one ulp each; 1/1 is exact,
// so silu(g) = g wherever e^-g is below half an ulp of 1, g > 16.7)
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}

// Per-token FP8 row scale of a gathered row (the scale of the token its
// sorted slot reads; 1 for padding slots, which are never stored).
__device__ __forceinline__ float gathered_row_scale(const GemmParams& p, int64_t row) {
  if (row >= p.m) return 1.0f;
  const int32_t f = p.sorted[row];
  return f < p.sentinel ? reinterpret_cast<const float*>(p.a_scale)[f / p.topk] : 1.0f;
}

// The per-token FP8 activation scale of output row `row` (1 for other
// formats): the row's own, or for gathered rows the gathered token's.
// AM: the row mode when known at compile time, -1 for the run-time flag
// (split-K reduce).
template <int FMT, int AM = -1>
__device__ __forceinline__ float row_act_scale(const GemmParams& p, int64_t row) {
  if (FMT != F_FP8) return 1.0f;
  const bool gathered = AM < 0 ? p.a_gather != 0 : AM == A_GATHER;
  return gathered ? gathered_row_scale(p, row) : reinterpret_cast<const float*>(p.a_scale)[row];
}

// Column scale of the plain / scatter epilogues (per-channel FP8 scale and
// the second-level scale); the per-token FP8 row scale is applied apart.
template <int FMT>
__device__ __forceinline__ float col_scale(const uint8_t* wmeta, int64_t col, float gs) {
  if (FMT == F_FP8 || fmt_w8_bf16(FMT)) return gs * reinterpret_cast<const float*>(wmeta)[col];
  return gs;
}

// Stores of one 16x16 accumulator tile held in the MFMA C layout (lane holds
// rows 4*lg + i of column c16) for the plain and scatter epilogues.  lrs:
// the tile's per-token FP8 row scales where the kernel computed them itself
// (row_base + r at lrs[r]), else null.
template <int FMT, int EPI, int AMODE>
__device__ __forceinline__ void store_tile(const GemmParams& p, const uint8_t* wmeta, float gs, int64_t row_base,
                                           int64_t col, const f32x4_t& v, int lg, const float* lrs = nullptr) {
  if (col >= p.n) return;
  uint16_t* out = static_cast<uint16_t*>(p.out);
  const float cs = col_scale<FMT>(wmeta, col, gs);
  const float bias = (EPI == EPI_BF16 && p.bias) ? bf16_bits_to_f32(p.bias[col]) : 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row_base + 4 * lg + i;
    if (row >= p.m) continue;
    float x = v[i] * cs;
    if (FMT == F_FP8) x *= lrs ? lrs[4 * lg + i] : row_act_scale<FMT, AMODE>(p, row);
    x += bias;
    if (EPI == EPI_SCATTER) {
      const int32_t f = p.sorted[row];
      if (f >= p.sentinel) continue;
      out[(int64_t)f * p.ldo + col] = (uint16_t)f32_to_bf16_bits(x);
    } else {
      // grouped rows in sorted order: padding slots are not stored
      if (AMODE != A_DIRECT && p.sorted[row] >= p.sentinel) continue;
      out[row * p.ldo + col] = (uint16_t)f32_to_bf16_bits(x);
    }
  }
}

// SwiGLU of one row's gate / up pair (columns col and col + I of the fused
// weight): a = silu(g) * u with the per-channel / second-level scales of
// either column and, for per-token FP8 activations, the row's scale.
template <int FMT>
__device__ __forceinline__ float swiglu_val(const GemmParams& p, const uint8_t* wmeta, float gs, float rs,
                                            int64_t col, float g, float u) {
  const float cg = col_scale<FMT>(wmeta, col, gs) * rs;
  const float cu = col_scale<FMT>(wmeta, col + p.n, gs) * rs;
  return silu_f32(g * cg) * (u * cu);
}

// The fp32 SwiGLU values an epilogue stores or requantizes, kept on request
// (stage export: the requantization's exact input), [rows][I].
__device__ __forceinline__ void keep_swiglu_f32(const GemmParams& p, int64_t row, int64_t col, float a) {
  if (p.swiglu_f32 && row < p.m && col < p.n) p.swiglu_f32[row * p.n + col] = a;
}

// SwiGLU epilogue of a gate / up tile pair in the C layout.
template <int FMT, int AMODE>
__device__ __forceinline__ void store_swiglu_bf16(const GemmParams& p, const uint8_t* wmeta, float gs, int64_t row_base,
                                                  int64_t col, const f32x4_t& g, const f32x4_t& u, int lg) {
  if (col >= p.n) return;
  uint16_t* out = static_cast<uint16_t*>(p.out);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row_base + 4 * lg + i;
    if (row >= p.m) continue;
    const float a = swiglu_val<FMT>(p, wmeta, gs, row_act_scale<FMT, AMODE>(p, row), col, g[i], u[i]);
    keep_swiglu_f32(p, row, col, a);
    out[row * p.ldo + col] = (uint16_t)f32_to_bf16_bits(a);
  }
}

// SwiGLU + MXFP8 requantization of 32 columns: two gate / up tile pairs.
// The 16 lanes of a DPP row hold the 16 columns of the same 4 rows, so the
// block absolute maximum is a row reduction.
template <int FMT>
__device__ __forceinline__ void store_swiglu_mxfp8(const GemmParams& p, const uint8_t* wmeta, float gs,
                                                   int64_t row_base, int64_t col0, const f32x4_t& g0,
                                                   const f32x4_t& u0, const f32x4_t& g1, const f32x4_t& u1, int lg,
                                                   int c16) {
  uint8_t* outq = static_cast<uint8_t*>(p.out);
  uint8_t* outs = static_cast<uint8_t*>(p.out_scale);
  const bool ok = (col0 - c16) < p.n;  // whole 32-column block valid (I % 32 == 0)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row_base + 4 * lg + i;
    const float a0 = swiglu_val<FMT>(p, wmeta, gs, 1.0f, col0, g0[i], u0[i]);
    const float a1 = swiglu_val<FMT>(p, wmeta, gs, 1.0f, col0 + 16, g1[i], u1[i]);
    if (ok) {
      keep_swiglu_f32(p, row, col0, a0);
      keep_swiglu_f32(p, row, col0 + 16, a1);
    }
    const float amax = row16_max(__builtin_fmaxf(__builtin_fabsf(a0), __builtin_fabsf(a1)));
    const int e = mx_scale_code(amax);
    const float inv = mx_inv_scale(e);
    const uint32_t q = f32x2_to_e4m3x2(a0 * inv, a1 * inv);
    if (ok && row < p.m) {
      outq[row * p.ldo + col0] = (uint8_t)(q & 0xFF);
      outq[row * p.ldo + col0 + 16] = (uint8_t)(q >> 8);
      if (c16 == 0) outs[row * (p.ldo / 32) + (col0 - c16) / 32] = (uint8_t)e;
    }
  }
}

// SwiGLU + MXFP4 requantization of 32 columns (W4A4): as the MXFP8 one,
// with E2M1 codes two per byte (even column in the low nibble): the lane of
// an even column takes its odd neighbour's code across the DPP quad and
// stores the byte.
template <int FMT>
__device__ __forceinline__ void store_swiglu_mxfp4(const GemmParams& p, const uint8_t* wmeta, float gs,
                                                   int64_t row_base, int64_t col0, const f32x4_t& g0,
                                                   const f32x4_t& u0, const f32x4_t& g1, const f32x4_t& u1, int lg,
                                                   int c16) {
  uint8_t* outq = static_cast<uint8_t*>(p.out);
  uint8_t* outs = static_cast<uint8_t*>(p.out_scale);
  const bool ok = (col0 - c16) < p.n;  // whole 32-column block valid (I % 32 == 0)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row_base + 4 * lg + i;
    const float a0 = swiglu_val<FMT>(p, wmeta, gs, 1.0f, col0, g0[i], u0[i]);
    const float a1 = swiglu_val<FMT>(p, wmeta, gs, 1.0f, col0 + 16, g1[i], u1[i]);
    if (ok) {
      keep_swiglu_f32(p, row, col0, a0);
      keep_swiglu_f32(p, row, col0 + 16, a1);
    }
    const float amax = row16_max(__builtin_fmaxf(__builtin_fabsf(a0), __builtin_fabsf(a1)));
    const int e = mx_scale_code_emax(amax, 2);
    const float inv = mx_inv_scale(e);
    const uint32_t q0 = f32_to_e2m1(a0 * inv), q1 = f32_to_e2m1(a1 * inv);
    const uint32_t n0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)q0, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    const uint32_t n1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)q1, 0xB1, 0xF, 0xF, false);
    if (ok && row < p.m && (c16 & 1) == 0) {
      uint8_t* rq = outq + row * (p.ldo / 2);
      rq[col0 / 2] = (uint8_t)(q0 | (n0 << 4));
      rq[(col0 + 16) / 2] = (uint8_t)(q1 | (n1 << 4));
      if (c16 == 0) outs[row * (p.ldo / 32) + (col0 - c16) / 32] = (uint8_t)e;
    }
  }
}

// Partial tile (fp32, natural [split][row][col] layout) of one 16x16 C tile.
__device__ __forceinline__ void store_partial(const GemmParams& p, int split, int64_t row_base, int64_t col,
                                              int64_t ncols, const f32x4_t& v, int lg) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row_base + 4 * lg + i;
    if (row >= p.m) continue;
    if (p.sorted && p.sorted[row] >= p.sentinel) continue;
    p.partials[((int64_t)split * p.m + row) * ncols + col] = v[i];
  }
}

// ---------------------------------------------------------------------------
// Decode kernel: one 16-row tile (at most 16 valid rows) of WN 16-column
// sub-tiles, KW compute waves splitting the workgroup's K range.
//
// The activation rows of the K range and the weight metadata (scales, zero
// points, E8M0 rows) are staged in LDS; each wave's only other loads are
// its weight ring, PF K-blocks deep, whose slots it consumes as they land
// (vector-memory loads complete in order).  Dense workgroups stage wave by
// wave (each wave copies its own contiguous K-blocks with plain loads issued
// ahead of its ring); MoE workgroups gather their rows through a loader wave
// with LDS-DMA.  Rows >= the valid count are never stored; their fragments
// repeat row 0 (an output row depends on its own A row alone).  LDS row
// layout per K-block: 16-byte chunks XOR-swizzled with the row, so the 16
// rows of one fragment read hit 16 different bank groups.  The KW partial
// sums are added in a fixed order through LDS at the end.

template <int FMT>
struct StreamLds {
  static constexpr int kRowB = 128 * Tr<FMT>::kAElem;  // bytes per row per K-block
};

// Waves of a stream workgroup: KW compute waves, plus a loader wave where
// the activation rows are gathered (MoE).  Dense workgroups stage their
// activations wave by wave and need none.
// (MXFP8 activations carry per-32 scales, which the loader wave stages.)
constexpr bool stream_self_staged(int fmt, int amode, int epi) {
  return amode == A_DIRECT && epi == EPI_BF16 && fmt != F_MXFP4_MXFP8;
}
constexpr int stream_waves(int fmt, int kw, int amode, int epi) {
  return kw + (stream_self_staged(fmt, amode, epi) ? 0 : 1);
}

// Decode-size routing of one 16-row expert block, run by each wave on its
// own (no barrier, no LDS): lane f holds flat slot f < route_n <= 64.  The
// lanes of one expert find each other with one ballot per id bit; a slot's
// position is its expert's padded segment start (the padded sizes of the
// smaller experts present) plus the number of earlier lanes of that expert,
// which is the align's stable order.  Returns the block's expert (-1: past
// the live blocks); lane r < 16 gets the slot of block row r (-1: padding);
// total = the padded live row count.  Slots routed outside [0, route_e) take
// no row, as in the align.
__device__ __forceinline__ int route_block(const GemmParams& p, int tm, int lane, int& slot, int& total) {
  const int n = p.route_n;
  int e = lane < n ? p.route_ids[lane] : -1;
  if (e < 0 || e >= p.route_e) e = -1;
  int nbits = 1;
  while ((1 << nbits) <= p.route_e) ++nbits;
  const uint32_t key = (uint32_t)(e + 1);
  uint64_t same = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t bal = __ballot(bit);
    same &= bit ? bal : ~bal;
  }
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(same & lt_mask);
  const int psz = e >= 0 ? (__popcll(same) + 15) / 16 * 16 : 0;
  const int lead = (e >= 0 && rank == 0) ? psz : 0;  // an expert's padded size, on its first lane
  int off = 0, tot = 0;
  for (int j = 0; j < n; ++j) {
    const int ej = __builtin_amdgcn_readlane(e, j);
    const int pj = __builtin_amdgcn_readlane(lead, j);
    off += ej < e ? pj : 0;
    tot += pj;
  }
  total = tot;
  const int base = tm * 16;
  const int pos = off + rank;
  const uint64_t own = __ballot(e >= 0 && off <= base && base < off + psz);
  const int expert = own ? __builtin_amdgcn_readlane(e, (int)__builtin_ctzll(own)) : -1;
  slot = -1;
  for (int r = 0; r < 16; ++r) {
    const uint64_t hit = __ballot(e >= 0 && pos == base + r);
    if (lane == r && hit) slot = (int)__builtin_ctzll(hit);
  }
  return expert;
}

template <int FMT, int WN, int KW, int PF, int AMODE, int EPI>
__global__ __launch_bounds__(64 * stream_waves(FMT, KW, AMODE, EPI)) void stream_kernel(const GemmParams p) {
  using T = Tr<FMT>;
  constexpr bool kSwiglu = (EPI == EPI_SWIGLU_BF16 || EPI == EPI_SWIGLU_MXFP8 || EPI == EPI_SWIGLU_MXFP4);
  // (W4A4 at decode sizes runs here as E4M3 x E2M1: its MXFP4 activations are
  // handed over as the E4M3 bytes of the same values, and the SwiGLU output
  // is requantized to MXFP4 for the W4A4 down GEMM)
  static_assert(FMT != F_MXFP4_MXFP4 && (EPI != EPI_SWIGLU_MXFP4 || FMT == F_MXFP4_MXFP8),
                "W4A4 decode: E4M3 x E2M1 with the MXFP4 SwiGLU epilogue");
  static_assert(!kSwiglu || WN % 2 == 0, "gate/up pairs");
  static_assert((EPI != EPI_SWIGLU_MXFP8 && EPI != EPI_SWIGLU_MXFP4) || WN % 4 == 0, "32-column MX blocks");
  constexpr int kRowB = StreamLds<FMT>::kRowB;
  constexpr int kCPR = kRowB / 16;
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  __shared__ int s_nrows;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, lg = lane >> 4;

  // grid (n-tile, m-tile, split): no index arithmetic
  const int tn = (int)blockIdx.x;
  const int tm = (int)blockIdx.y;
  const int split = (int)blockIdx.z;

  int expert = 0;
  int route_slot = -1;  // routing inside the kernel: the slot of tile row `lane` (lanes < 16)
  if constexpr (AMODE != A_DIRECT || EPI == EPI_SCATTER) {  // grouped rows: the block's expert (-1: all padding)
    if (AMODE == A_GATHER && p.route_ids) {
      int total = 0;
      expert = route_block(p, tm, lane, route_slot, total);
      // the routing of every launched block, for the GEMM after this one
      if (tn == 0 && split == 0 && wave == 0) {
        if (lane < 16 && (int64_t)tm * 16 + lane < p.m)
          p.route_sorted[tm * 16 + lane] = route_slot >= 0 ? route_slot : p.sentinel;
        if (lane == 0) p.route_bexp[tm] = expert;
        if (lane == 0 && tm == 0) *p.route_live = total;
      }
    } else {
      expert = p.block_expert[tm];
    }
    if (expert < 0) return;
  }
  const int64_t row0 = tm * 16;
  WPtrs wp;
  wp.codes = p.codes + (int64_t)expert * p.codes_per_expert;
  wp.meta = p.wscale + (int64_t)expert * p.scales_per_expert;
  // without zero points the (unused) zero loads read the scale array
  wp.zero = p.wzero ? p.wzero + (int64_t)expert * p.zeros_per_expert : wp.meta;
  const float gs = p.gscale[expert];

  int nts[WN];
  bool ntv[WN];
#pragma unroll
  for (int ns = 0; ns < WN; ++ns) {
    if constexpr (kSwiglu) {
      const int ntg = tn * (WN / 2) + ns % (WN / 2);
      ntv[ns] = ntg * 16 < p.n;
      nts[ns] = ntg + (ns >= WN / 2 ? p.swiglu_nt_off : 0);
    } else {
      nts[ns] = tn * WN + ns;
      ntv[ns] = nts[ns] < p.nt_count;
    }
  }

  const int kb_begin = split * p.kb_per_split;
  int kb_end = kb_begin + p.kb_per_split;
  if (kb_end > p.kb_count) kb_end = p.kb_count;
  const int nkb = kb_end > kb_begin ? kb_end - kb_begin : 0;
  constexpr bool kSelf = stream_self_staged(FMT, AMODE, EPI);
  // Self-staged (dense) workgroups give compute wave w the contiguous
  // K-blocks [kw0, kw0 + nj); otherwise wave w takes kb_begin + w, + KW, ...
  // (wave KW, the loader, takes none).
  int kw0, nj;
  if constexpr (kSelf) {
    const int per = (nkb + KW - 1) / KW;
    kw0 = kb_begin + wave * per;
    const int kw1 = kw0 + per < kb_end ? kw0 + per : kb_end;
    nj = kw1 > kw0 ? kw1 - kw0 : 0;
  } else {
    kw0 = kb_begin + wave;
    nj = (wave < KW && kw0 < kb_end) ? (kb_end - kw0 + KW - 1) / KW : 0;
  }
  // the wave's j-th K-block (j < nj + PF; it matters only for j < nj)
  auto kb_at = [&](int j) { return kSelf ? kw0 + j : kw0 + j * KW; };

  // The loader wave finds the source row of each tile row (-1: padding /
  // past the end) and stages the activation rows of the K range into LDS
  // with LDS-DMA loads; the compute waves issue their weight rings (the
  // loader's range is empty, so its ring loads return zeros at once).
  WStripe st[WN];
#pragma unroll
  for (int ns = 0; ns < WN; ++ns) st[ns] = make_stripe<FMT>(p, wp, nts[ns], ntv[ns]);
  // first scale group / first 4-K-block E8M0 row of the K range (the LDS
  // metadata starts there)
  const int g0 = fmt_int(FMT) ? kb_begin / p.kb_per_group : 0;
  constexpr int kRS = T::kMetaRowShift;
  const int r0 = kb_begin >> kRS;
  auto stage = [&]() {
    // source row of tile row `lane` (lanes 0..15; -1: padding / past the end)
    int src = -1;
    if (lane < 16) {
      const int64_t row = row0 + lane;
      if (AMODE == A_GATHER) {
        if (p.route_ids) {
          if (route_slot >= 0) src = route_slot / p.topk;
        } else {
          const int32_t f = row < p.m ? p.sorted[row] : p.sentinel;
          if (f < p.sentinel) src = f / p.topk;
        }
      } else if (row < p.m) {
        // grouped rows in sorted order: padding slots (sentinel) are skipped
        src = (p.sorted && p.sorted[row] >= p.sentinel) ? -1 : (int)row;
      }
    }
    // rows [0, nr) are stored (dense: rows < m are a prefix; MoE: the valid
    // rows of a block are a prefix).  Direct rows are row0 + r; gathered
    // ones are read from lane r.
    const int nr = __builtin_popcountll(__builtin_amdgcn_ballot_w64(src >= 0));
    if (lane == 0) s_nrows = nr;
    if (nr == 0) return;
    auto src_row = [&](int r) -> int64_t {
      if constexpr (AMODE == A_GATHER) return __builtin_amdgcn_ds_bpermute(r << 2, src);
      return row0 + r;
    };
    // x / nr for x < 2^14 (nr <= 16) as a multiply-shift: exact while
    // x * nr < 2^20
    const uint32_t mnr = ((1u << 20) + nr - 1) / nr;
    // LDS: activation slots (rounded up to whole 64-lane DMA instructions),
    // then the MX scale dwords (likewise rounded).  Each DMA instruction
    // fills 64 consecutive 16-byte slots; slot s of the layout
    // [K-block][row][swizzled chunk] holds logical chunk phys ^ swizzle(row).
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.a, p.a_bytes);
    const int slots = nr * kCPR * nkb;
#pragma unroll 1
    for (int base = 0; base < slots; base += 64) {
      const int sidx = base + lane;
      const int phys = sidx & (kCPR - 1);
      const uint32_t rowkb = (uint32_t)sidx / kCPR;
      const int kbl = (int)((rowkb * mnr) >> 20);
      const int r = (int)rowkb - kbl * nr;
      const int c = T::kBf16 ? (phys ^ r) : (phys ^ ((r >> 1) & 7));
      const int64_t sr = src_row(r < nr ? r : 0);
      // lanes past `slots` fill unused slots of the footprint from offset 0
      // (always a valid address): no reliance on range checking
      const uint32_t voff = sidx < slots
                                ? (uint32_t)((sr * p.lda + (int64_t)(kb_begin + kbl) * 128) * T::kAElem + c * 16)
                                : 0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dsm + base * 16, 16, voff, 0, 0, 0);
    }
    if (FMT == F_MXFP4_MXFP8) {
      const int scale_off = ((slots + 63) & ~63) * 16;
      const __amdgpu_buffer_rsrc_t rsc = make_rsrc(p.a_scale, p.a_scale_bytes);
      const int n4 = nr * nkb;
#pragma unroll 1
      for (int base = 0; base < n4; base += 64) {
        const int sidx = base + lane;
        const int kbl = (int)(((uint32_t)sidx * mnr) >> 20);
        const int r = sidx - kbl * nr;
        const int64_t sr = src_row(r < nr ? r : 0);
        const uint32_t voff = sidx < n4 ? (uint32_t)(sr * p.a_scale_ld + (int64_t)(kb_begin + kbl) * 4) : 0u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, dsm + scale_off + base * 4, 4, voff, 0, 0, 0);
      }
    }
    // weight metadata of the K range, per valid sub-tile (filler lanes read
    // the stripe's first bytes, which always exist)
    if (fmt_int(FMT) && nkb > 0) {
      const int g1 = (kb_end - 1) / p.kb_per_group + 1;
      const int ss = p.scale_f32 ? 4 : 2;
      const int n16 = (g1 - g0) * ss;  // 16-byte slots of scales
      const int n4 = (g1 - g0) * 2;    // 4-byte slots of zero points
#pragma unroll
      for (int ns = 0; ns < WN; ++ns) {
        if (!ntv[ns]) continue;
        uint8_t* mb = dsm + p.lds_meta_off + ns * p.lds_meta_stride;
        // (resources copied to locals: a captured array member passed to
        // the LDS-DMA builtin makes the host pass drop the kernel's stub)
        const __amdgpu_buffer_rsrc_t rm = st[ns].meta, rz = st[ns].zero;
#pragma unroll 1
        for (int base = 0; base < n16; base += 64) {
          const int sl = base + lane;
          const uint32_t voff = sl < n16 ? (uint32_t)(g0 * 16 * ss + sl * 16) : 0u;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rm, mb + base * 16, 16, voff, 0, 0, 0);
        }
        if (p.has_zero) {
#pragma unroll 1
          for (int base = 0; base < n4; base += 64) {
            const int sl = base + lane;
            const uint32_t voff = sl < n4 ? (uint32_t)(g0 * 8 + sl * 4) : 0u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, mb + p.lds_zero_off + base * 4, 4, voff, 0, 0, 0);
          }
        }
      }
    } else if ((fmt_mx_meta(FMT)) && nkb > 0) {
      const int n16 = (((kb_end + (1 << kRS) - 1) >> kRS) - r0) * 16;  // 16-byte slots of scale rows
#pragma unroll
      for (int ns = 0; ns < WN; ++ns) {
        if (!ntv[ns]) continue;
        uint8_t* mb = dsm + p.lds_meta_off + ns * p.lds_meta_stride;
        const __amdgpu_buffer_rsrc_t rm = st[ns].meta;
#pragma unroll 1
        for (int base = 0; base < n16; base += 64) {
          const int sl = base + lane;
          const uint32_t voff = sl < n16 ? (uint32_t)(r0 * 256 + sl * 16) : 0u;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rm, mb + base * 16, 16, voff, 0, 0, 0);
        }
      }
    }
  };
  BFrag<FMT> ring[PF][WN];
  auto issue_ring = [&]() {
#pragma unroll
    for (int q = 0; q < PF; ++q) {
#pragma unroll
      for (int ns = 0; ns < WN; ++ns) ring[q][ns] = load_b<FMT, false>(p, st[ns], q < nj, kb_at(q), lane);
      // issue slot by slot, in the order of use (they land in issue order)
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Loader path (gathered rows): the rings go out first, the loader wave
  // looks the rows up and DMAs them, and waits for its DMA inside its own
  // branch (the compiler waits for every outstanding vector-memory load
  // before an LDS read that follows an LDS-DMA it cannot prove finished, so
  // the wait must close the branch).
  auto stage_via_loader = [&]() {
    issue_ring();
    if (wave == KW) {
      stage();
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
  };
  auto self_stage = [&](int nr) {
    const int nch = nj * nr * kCPR;                  // 16-byte activation chunks (<= 512)
    const int slot0 = (kw0 - kb_begin) * nr * kCPR;  // first LDS slot of the wave's K-blocks
    const uint32_t mnr = ((1u << 20) + nr - 1) / nr; // x / nr as a multiply-shift (x * nr < 2^20)
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
    u32x4_t abuf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i * 64 + lane;
      const uint32_t rowkb = (uint32_t)c / kCPR;
      const int kbl = (int)((rowkb * mnr) >> 20);
      const int r = (int)rowkb - kbl * nr;
      const int phys = c & (kCPR - 1);
      const int lc = T::kBf16 ? (phys ^ r) : (phys ^ ((r >> 1) & 7));
      const uint32_t off = (uint32_t)(((row0 + r) * p.lda + (int64_t)(kw0 + kbl) * 128) * T::kAElem + lc * 16);
      abuf[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, c < nch ? off : kOob, 0, 0);
    }
    // weight metadata of the wave's K-blocks (INT: scales and zero points of
    // the groups they touch; MX: their 4-K-block E8M0 rows), up to kML KB
    constexpr int kML =
        fmt_int(FMT) ? 1 : ((fmt_mx_meta(FMT)) ? 2 : 0);
    u32x4_t mbuf[WN][kML > 0 ? kML : 1];
    uint32_t zbuf[WN];
    int mb0 = 0, mbytes = 0, zb0 = 0, zbytes = 0, mdst = 0, zdst = 0;
    if (fmt_int(FMT) && nj > 0) {
      const int g0w = kw0 / p.kb_per_group, g1w = (kw0 + nj - 1) / p.kb_per_group + 1;
      const int ss = p.scale_f32 ? 4 : 2;
      mb0 = g0w * 16 * ss;
      mbytes = (g1w - g0w) * 16 * ss;  // <= 1 KB
      mdst = (g0w - g0) * 16 * ss;
      zb0 = g0w * 8;
      zbytes = p.has_zero ? (g1w - g0w) * 8 : 0;  // <= 256 B
      zdst = p.lds_zero_off + (g0w - g0) * 8;
    } else if ((fmt_mx_meta(FMT)) && nj > 0) {
      const int rw0 = kw0 >> kRS, rw1 = (kw0 + nj + (1 << kRS) - 1) >> kRS;
      mb0 = rw0 * 256;
      mbytes = (rw1 - rw0) * 256;  // <= 2 KB
      mdst = (rw0 - r0) * 256;
    }
#pragma unroll
    for (int ns = 0; ns < WN; ++ns) {
#pragma unroll
      for (int i = 0; i < kML; ++i) {
        const int b = (i * 64 + lane) * 16;
        mbuf[ns][i] = __builtin_amdgcn_raw_buffer_load_b128(st[ns].meta, b < mbytes ? (uint32_t)(mb0 + b) : kOob, 0, 0);
      }
      if (fmt_int(FMT))
        zbuf[ns] = __builtin_amdgcn_raw_buffer_load_b32(st[ns].zero,
                                                        lane * 4 < zbytes ? (uint32_t)(zb0 + lane * 4) : kOob, 0, 0);
    }
    issue_ring();
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i * 64 + lane < nch) *reinterpret_cast<u32x4_t*>(dsm + (slot0 + i * 64 + lane) * 16) = abuf[i];
#pragma unroll
    for (int ns = 0; ns < WN; ++ns) {
      uint8_t* mb = dsm + p.lds_meta_off + ns * p.lds_meta_stride;
#pragma unroll
      for (int i = 0; i < kML; ++i)
        if ((i * 64 + lane) * 16 < mbytes) *reinterpret_cast<u32x4_t*>(mb + mdst + (i * 64 + lane) * 16) = mbuf[ns][i];
      if (fmt_int(FMT) && lane * 4 < zbytes) *reinterpret_cast<uint32_t*>(mb + zdst + lane * 4) = zbuf[ns];
    }
  };

  // Per-token FP8 activations quantized here (dense decode, p.a_fp8_fuse: p.a
  // holds the bf16 rows).  The rule is the activation quantizer's: s = amax /
  // 448 over the whole row (1 for an all-zero row), codes E4M3 round to
  // nearest even of x / s, saturated.  Each wave loads the bf16 values of its
  // own K-blocks (the chunks its code slots hold), issues its ring, and posts
  // each row's maximum over them (a max over the 8 lanes of a chunk row, then
  // an LDS max, order free); after one LDS-only barrier every wave takes the
  // row maxima of all waves, divides, converts and writes its code slots.
  // The codes and scales are the quantizer's bit for bit, so the result is
  // that of the two-launch path.
  constexpr bool kFuse = (FMT == F_FP8 || FMT == F_FP8_BLOCK) && kSelf;
  constexpr bool kBlk = FMT == F_FP8_BLOCK && kSelf;
  constexpr int kFuseCh = 4;  // code chunks per lane (a wave's K range holds at most 256)
  __shared__ uint32_t s_amax[FMT == F_FP8 && kSelf ? KW * 16 : 1];
  __shared__ float s_rsc[FMT == F_FP8 && kSelf ? 16 : 1];
  auto fuse_stage = [&](int nr) {
    const int nch = nj * nr * kCPR;                  // 16-byte code chunks (<= 256)
    const int slot0 = (kw0 - kb_begin) * nr * kCPR;
    const uint32_t mnr = ((1u << 20) + nr - 1) / nr;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
    u32x4_t xb[2 * kFuseCh];
    int rw[kFuseCh];
#pragma unroll
    for (int i = 0; i < kFuseCh; ++i) {
      const int c = i * 64 + lane;
      const uint32_t rowkb = (uint32_t)c / kCPR;
      const int kbl = (int)((rowkb * mnr) >> 20);
      const int r = (int)rowkb - kbl * nr;
      const int lc = (c & (kCPR - 1)) ^ ((r >> 1) & 7);
      rw[i] = r < 16 ? r : 0;
      const uint32_t off = (uint32_t)(((row0 + r) * p.lda + (int64_t)(kw0 + kbl) * 128 + lc * 16) * 2);
      xb[2 * i] = __builtin_amdgcn_raw_buffer_load_b128(ra, c < nch ? off : kOob, 0, 0);
      xb[2 * i + 1] = __builtin_amdgcn_raw_buffer_load_b128(ra, c < nch ? off + 16 : kOob, 0, 0);
    }
    if constexpr (kBlk) {
      // block-scaled FP8: the scale group of a chunk is its row's K-block,
      // whose 8 chunks are the 8 lanes of a chunk row: the group's maximum
      // is a reduction over them, no other wave is involved.  The group
      // scales go to [K-block][16 rows] after the code slots, the sub-tiles'
      // block scales of the wave's K-blocks to [K-block][WN] after them.
      const int sa_off = ((nr * kCPR * nkb + 63) & ~63) * 16;
      const int sw_off = sa_off + nkb * 64;
      // (at most 4 code chunks per lane: a wave's K range is at most 32
      // K-blocks, so its WN <= 4 sub-tiles hold at most 128 block scales)
      const int nsw = nj * WN;
      const __amdgpu_buffer_rsrc_t rm = make_rsrc(wp.meta, p.scales_per_expert);
      float swv[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = h * 64 + lane, ns = e % WN, j = e / WN;
        const uint32_t mo = (e < nsw && ntv[ns]) ? (uint32_t)((nts[ns] * (int64_t)p.kb_count + kw0 + j) * 4) : kOob;
        swv[h] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rm, mo, 0, 0));
      }
      issue_ring();
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = h * 64 + lane;
        if (e < nsw) *reinterpret_cast<float*>(dsm + sw_off + ((kw0 - kb_begin + e / WN) * WN + e % WN) * 4) = swv[h];
      }
#pragma unroll
      for (int i = 0; i < kFuseCh; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        const int c = i * 64 + lane;
        float mx = 0.0f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            mx = __builtin_fmaxf(mx, __builtin_fabsf(bf16_bits_to_f32(xb[2 * i + h][d] & 0xFFFF)));
            mx = __builtin_fmaxf(mx, __builtin_fabsf(bf16_bits_to_f32(xb[2 * i + h][d] >> 16)));
          }
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 1));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 2));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 4));
        if (c >= nch) continue;
        const float sc = mx > 0.0f ? mx / 448.0f : 1.0f;  // IEEE f32 division
        const uint32_t rowkb = (uint32_t)c / kCPR;
        const int kbl = (int)((rowkb * mnr) >> 20);
        if ((lane & 7) == 0)
          *reinterpret_cast<float*>(dsm + sa_off + ((kw0 - kb_begin + kbl) * 16 + rw[i]) * 4) = sc;
        u32x4_t q;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const uint32_t w0 = xb[2 * i + h][2 * d], w1 = xb[2 * i + h][2 * d + 1];
            q[2 * h + d] = f32x2_to_e4m3x2(bf16_bits_to_f32(w0 & 0xFFFF) / sc, bf16_bits_to_f32(w0 >> 16) / sc) |
                           (f32x2_to_e4m3x2(bf16_bits_to_f32(w1 & 0xFFFF) / sc, bf16_bits_to_f32(w1 >> 16) / sc) << 16);
          }
        *reinterpret_cast<u32x4_t*>(dsm + (slot0 + c) * 16) = q;
      }
      return;
    }
    issue_ring();
    uint32_t* am = s_amax + wave * 16;
    if (lane < 16) am[lane] = 0u;  // (a wave's LDS accesses complete in order)
#pragma unroll
    for (int i = 0; i < kFuseCh; ++i) {
      float mx = 0.0f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          mx = __builtin_fmaxf(mx, __builtin_fabsf(bf16_bits_to_f32(xb[2 * i + h][d] & 0xFFFF)));
          mx = __builtin_fmaxf(mx, __builtin_fabsf(bf16_bits_to_f32(xb[2 * i + h][d] >> 16)));
        }
      // the 8 lanes of one chunk row (c / 8) share its row
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 1));
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 2));
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 4));
      if ((lane & 7) == 0 && i * 64 + lane < nch) atomicMax(&am[rw[i]], __float_as_uint(mx));
    }
    // every wave's maxima posted (LDS only: the ring stays in flight)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    auto row_scale = [&](int r) -> float {
      uint32_t u = 0;
#pragma unroll
      for (int w = 0; w < KW; ++w) u = u > s_amax[w * 16 + r] ? u : s_amax[w * 16 + r];
      const float amax = __uint_as_float(u);
      return amax > 0.0f ? amax / 448.0f : 1.0f;  // IEEE f32 division
    };
    if (wave == 0 && lane < 16) s_rsc[lane] = row_scale(lane);
#pragma unroll
    for (int i = 0; i < kFuseCh; ++i) {
      // (one chunk at a time: the divisions of all chunks at once would hold
      // far more registers than the decode loop)
      __builtin_amdgcn_sched_barrier(0);
      const int c = i * 64 + lane;
      if (c >= nch) continue;
      const float sc = row_scale(rw[i]);
      u32x4_t q;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const uint32_t w0 = xb[2 * i + h][2 * d], w1 = xb[2 * i + h][2 * d + 1];
          q[2 * h + d] = f32x2_to_e4m3x2(bf16_bits_to_f32(w0 & 0xFFFF) / sc, bf16_bits_to_f32(w0 >> 16) / sc) |
                         (f32x2_to_e4m3x2(bf16_bits_to_f32(w1 & 0xFFFF) / sc, bf16_bits_to_f32(w1 >> 16) / sc) << 16);
        }
      *reinterpret_cast<u32x4_t*>(dsm + (slot0 + c) * 16) = q;
    }
  };

  int nrows = 0;
  if constexpr (kSelf) {
    // Each wave copies the activation rows and weight metadata of its own
    // K-blocks into their places of the workgroup's LDS layout with plain
    // loads issued ahead of its ring (vector-memory loads land in issue
    // order, so the copy waits for them alone), then reads only what it
    // wrote: no barrier, no loader.  Rows < m of the tile are a prefix.
    nrows = p.m - row0 < 16 ? (int)(p.m - row0) : 16;
    if constexpr (kBlk) {
      fuse_stage(nrows);  // (block-scaled FP8 rows are always quantized here)
    } else if constexpr (kFuse) {
      if (p.a_fp8_fuse)
        fuse_stage(nrows);
      else
        self_stage(nrows);
    } else {
      self_stage(nrows);
    }
  } else {
    stage_via_loader();
    nrows = s_nrows;
  }

  const int scale_off = ((nrows * kCPR * nkb + 63) & ~63) * 16;

  f32x4_t acc[WN];
#pragma unroll
  for (int ns = 0; ns < WN; ++ns) acc[ns] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const bool arow_ok = c16 < nrows;
  const int rr = arow_ok ? c16 : 0;  // LDS row read (row 0 stands in for empty rows)
  const IntScaleSel ssel = int_scale_sel(p, c16);
  // raw metadata words of sub-tile ns at K-block kb, from the LDS copy
  auto lds_meta = [&](int ns, int kb, uint32_t& m, uint32_t& z) {
    const uint8_t* mb = dsm + p.lds_meta_off + ns * p.lds_meta_stride;
    m = 0;
    z = 0;
    if (fmt_int(FMT)) {
      const int gl = (int)(((float)kb + 0.5f) * p.inv_kbg) - g0;
      const int sf = p.scale_f32;
      m = *reinterpret_cast<const uint32_t*>(mb + ((gl * 16 + (c16 & (14 | sf))) << (1 + sf)));
      const uint32_t zr = *reinterpret_cast<const uint32_t*>(mb + p.lds_zero_off + gl * 8 + ((c16 >> 3) << 2));
      z = p.has_zero ? zr : 0u;
    } else if (fmt_mx_meta(FMT)) {
      m = *reinterpret_cast<const uint32_t*>(mb + (((kb >> kRS) - r0) * 64 + lane) * 4);
    }
  };

  for (int j0 = 0; j0 < nj; j0 += PF) {
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      const int j = j0 + q;
      if (j < nj) {
        const int kb = kb_at(j);
        const uint8_t* ab = dsm + ((kb - kb_begin) * nrows + rr) * kRowB;
        if constexpr (T::kBf16) {
          // (rows >= nrows read row 0: an output row depends on its own A
          // row alone, and those rows are never stored)
          bf16x8_t af[4];
#pragma unroll
          for (int s = 0; s < 4; ++s)
            af[s] = *reinterpret_cast<const bf16x8_t*>(ab + (((4 * lg + s) ^ rr) * 16));
          f32x4_t rs = {0.0f, 0.0f, 0.0f, 0.0f};
          if (fmt_int(FMT)) {
            // row sums of the K-block in the C layout: A x ones
            const u32x4_t o = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
            const bf16x8_t one = __builtin_bit_cast(bf16x8_t, o);
            const bf16x8_t on[4] = {one, one, one, one};
            rs = mfma_bf16_kblock(af, on, rs);
          }
#pragma unroll
          for (int ns = 0; ns < WN; ++ns) {
            bf16x8_t d[4];
            uint32_t mw, zw;
            lds_meta(ns, kb, mw, zw);
            dequant_b<FMT>(ring[q][ns], mw, kb, d);
            if (fmt_int(FMT)) {
              const f32x4_t t = mfma_bf16_kblock(af, d, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f});
              const float sc = frag_int_scale(mw, ssel);
              const float off = (float)(p.int_offset + frag_int_zero(zw, c16));
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[ns][i] = __builtin_fmaf(sc, __builtin_fmaf(-off, rs[i], t[i]), acc[ns][i]);
            } else {
              acc[ns] = mfma_bf16_kblock(af, d, acc[ns]);
            }
          }
        } else {
          const int sw = (rr >> 1) & 7;
          const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(ab + ((lg ^ sw) * 16));
          const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(ab + (((4 + lg) ^ sw) * 16));
          int sa = 127;
          if (FMT == F_MXFP4_MXFP8) {
            const uint32_t sw4 = reinterpret_cast<const uint32_t*>(dsm + scale_off)[(kb - kb_begin) * nrows + rr];
            sa = arow_ok ? (int)((sw4 >> (8 * lg)) & 0xFF) : 127;
          }
          i32x8_t a8;
          a8[0] = lo[0]; a8[1] = lo[1]; a8[2] = lo[2]; a8[3] = lo[3];
          a8[4] = hi[0]; a8[5] = hi[1]; a8[6] = hi[2]; a8[7] = hi[3];
          if constexpr (kBlk) {
            // acc += (row group scale x sub-tile block scale) x this K-block's sum
            const int sa_off = ((nrows * kCPR * nkb + 63) & ~63) * 16;
            const f32x4_t sg = *reinterpret_cast<const f32x4_t*>(dsm + sa_off + ((kb - kb_begin) * 16 + 4 * lg) * 4);
#pragma unroll
            for (int ns = 0; ns < WN; ++ns) {
              const float sw = *reinterpret_cast<const float*>(dsm + sa_off + nkb * 64 + ((kb - kb_begin) * WN + ns) * 4);
              const f32x4_t t = mfma_f8_kblock<FMT>(a8, 127, ring[q][ns], 0u, kb, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[ns][i] = __builtin_fmaf(sg[i] * sw, t[i], acc[ns][i]);
            }
          } else {
#pragma unroll
            for (int ns = 0; ns < WN; ++ns) {
              uint32_t mw, zw;
              lds_meta(ns, kb, mw, zw);
              acc[ns] = mfma_f8_kblock<FMT>(a8, sa, ring[q][ns], mw, kb, acc[ns]);
            }
          }
        }
      }
      // refill (past the end of the range the load returns zeros without
      // touching memory)
#pragma unroll
      for (int ns = 0; ns < WN; ++ns) ring[q][ns] = load_b<FMT, false>(p, st[ns], j + PF < nj, kb_at(j + PF), lane);
    }
  }

  // in-workgroup reduction over the KW waves (fixed order), through the LDS
  // that held the activations
  if constexpr (KW > 1) {
    f32x4_t* red = reinterpret_cast<f32x4_t*>(dsm);
    __syncthreads();
    if (wave > 0 && wave < KW) {
#pragma unroll
      for (int ns = 0; ns < WN; ++ns) red[((wave - 1) * WN + ns) * 64 + lane] = acc[ns];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 1; w < KW; ++w)
#pragma unroll
      for (int ns = 0; ns < WN; ++ns) {
        const f32x4_t v = red[((w - 1) * WN + ns) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[ns][i] += v[i];
      }
  }

  if (p.split_k > 1) {
    const int64_t ncols = kSwiglu ? 2 * p.n : (int64_t)p.nt_count * 16;
#pragma unroll
    for (int ns = 0; ns < WN; ++ns) {
      if (!ntv[ns]) continue;
      store_partial(p, split, row0, (int64_t)nts[ns] * 16 + c16, ncols, acc[ns], lg);
    }
    return;
  }
  if constexpr (EPI == EPI_BF16 || EPI == EPI_SCATTER) {
#pragma unroll
    for (int ns = 0; ns < WN; ++ns)
      store_tile<FMT, EPI, AMODE>(p, wp.meta, gs, row0, (int64_t)nts[ns] * 16 + c16, acc[ns], lg,
                                  (FMT == F_FP8 && kSelf && p.a_fp8_fuse) ? s_rsc : nullptr);
  } else if constexpr (EPI == EPI_SWIGLU_BF16) {
#pragma unroll
    for (int j = 0; j < WN / 2; ++j)
      store_swiglu_bf16<FMT, AMODE>(p, wp.meta, gs, row0, (int64_t)nts[j] * 16 + c16, acc[j], acc[j + WN / 2], lg);
  } else if constexpr (EPI == EPI_SWIGLU_MXFP4) {
#pragma unroll
    for (int jj = 0; jj < WN / 4; ++jj)
      store_swiglu_mxfp4<FMT>(p, wp.meta, gs, row0, (int64_t)nts[2 * jj] * 16 + c16, acc[2 * jj], acc[2 * jj + WN / 2],
                              acc[2 * jj + 1], acc[2 * jj + 1 + WN / 2], lg, c16);
  } else {
#pragma unroll
    for (int jj = 0; jj < WN / 4; ++jj)
      store_swiglu_mxfp8<FMT>(p, wp.meta, gs, row0, (int64_t)nts[2 * jj] * 16 + c16, acc[2 * jj], acc[2 * jj + WN / 2],
                         acc[2 * jj + 1], acc[2 * jj + 1 + WN / 2], lg, c16);
  }
}

// ---------------------------------------------------------------------------
// Prefill kernel: a (16 WM) x (64 WN) output tile per workgroup of 4 waves;
// wave w owns columns [16 WN w, 16 WN (w + 1)) of the tile for all its rows.
//
// Every K-block's activation tile (16 WM rows, 16-byte chunks XOR-swizzled
// with the row), with the MXFP8 scale words of its rows and each wave's
// metadata words (INT scale dwords or E8M0 rows), goes from global memory
// straight into LDS by LDS-DMA, kS - 1 K-blocks ahead of its use.  Each
// wave's weight-code fragments (private to the wave) go straight into
// registers, one register set per stage.  A K-block step is: issue the
// copies of K-block j + kS - 1, compute K-block j, wait until this wave's
// copies of K-block j + 1 have landed (with three stages the copies of
// K-block j + 2 stay in flight), barrier.  With two stages the LDS copies
// are issued from inline assembly, which the compiler does not track, and
// every step ends with a full wait; with three they are issued through the
// compiler's builtin into one LDS array per stage, so that the compiler's
// own waits for the register fragments count them too.

template <int FMT, int WM, int WN, int AMODE, int EPI, int S>
struct TileCfg {
  using T = Tr<FMT>;
  // pipeline stages (2 or 3): with two, a K-block's copy overlaps one
  // K-block of compute; with three it has two K-blocks of compute to land
  static constexpr int kS = S;
  static constexpr int kTM = 16 * WM;
  static constexpr int kTNS = 4 * WN;                            // weight sub-tiles per workgroup
  static constexpr int kRowB = T::kARowB;                        // activation bytes per row per K-block
  static constexpr int kCPR = kRowB / 16;                        // 16-byte chunks per row
  static constexpr int kA = kTM * kRowB;                         // activation tile (whole KB)
  static constexpr int kAI = kA / 1024;                          // its 1-KB DMA instructions
  static constexpr int kAIW = (kAI + 3) / 4;                     // ... per wave
  // a dword per row and K-block: MX scales (E8M0 per 32) or the f32 scale of
  // a per-group FP8 row
  static constexpr bool kX = (FMT == F_MXFP4_MXFP8 || FMT == F_MXFP4_MXFP4 || FMT == F_FP8_BLOCK);
  static constexpr int kXI = kX ? (kTM + 63) / 64 : 0;           // its 256-B DMA instructions
  static constexpr int kCB = 64 * T::kCodeB;                     // code bytes per sub-tile per K-block
  // Each wave loads its own weight fragments straight into registers,
  // kS - 1 K-blocks ahead, one register set per stage (they are private to
  // the wave: staging them through LDS would only add LDS traffic).
  static constexpr bool kBReg = true;
  static constexpr int kB = 0;
  // Three stages issue their LDS copies through the compiler's builtin, so
  // that its count of loads in flight includes them and its waits for the
  // register fragments (two stages deep) are exact; two stages issue them
  // from inline assembly and wait for everything at the end of each step.
  static constexpr bool kTracked = (kS == 3);
  static constexpr int kMI = (fmt_int(FMT) || FMT == F_FP8_BLOCK)
                                 ? 1
                                 : ((fmt_mx_meta(FMT) || FMT == F_MXFP4_MXFP4) ? WN : 0);
  static constexpr int kM = 4 * kMI * 256;                       // metadata words (per wave: kMI x 256 B)
  static constexpr int kStage = kA + kXI * 256 + kB + kM;
  static constexpr bool kSwiglu = (EPI == EPI_SWIGLU_BF16 || EPI == EPI_SWIGLU_MXFP8 || EPI == EPI_SWIGLU_MXFP4);
  static_assert(!kSwiglu || WN % 2 == 0, "gate/up pairs");
  static_assert((EPI != EPI_SWIGLU_MXFP8 && EPI != EPI_SWIGLU_MXFP4) || WN % 4 == 0, "32-column MX blocks");
  static_assert(kA % 1024 == 0, "whole 1-KB activation DMA instructions");
  static_assert(kS * kStage <= 160 * 1024, "LDS budget");
  static_assert(!fmt_int(FMT) || WN * 16 <= 64, "INT scale words of a wave fit one DMA instruction");
};

// Physical 16-byte chunk of logical chunk c of LDS tile row r, for rows of
// cpr chunks (16: bf16, 8: FP8, 4: FP4): the rows of one fragment read land
// on different banks.  bf16 rows take one of two XOR masks: for the 16x16
// fragment reads (a K-group's 16 lanes read 16 consecutive rows, one chunk)
// the row's bits 0-1 go to chunk bits 2-3 and bits 2-3 to chunk bits 0-1
// (measured on gfx950: no bank conflicts, against 3.9 conflict cycles per
// read with the row's low four bits XORed in unchanged, which the 32x32
// fragment reads of 32 rows keep, conflict-free for them).
__device__ __forceinline__ int swz(int r, int c, int cpr, bool rot16 = false) {
  const int r16 = r & 15;
  return cpr == 16 ? (c ^ (rot16 ? ((r16 >> 2) | ((r16 & 3) << 2)) : r16))
                   : (cpr == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3)));
}

// LDS of the pipeline: kS stages of kStage bytes, each holding the
// activation tile, the per-row words, the code fragments and the metadata
// words at fixed offsets.
template <int FMT, int WM, int WN, int AMODE, int EPI, int S>
struct TileLds {
  using C = TileCfg<FMT, WM, WN, AMODE, EPI, S>;
  // (three stages: one array each, so that the compiler can tell a copy
  // into one stage from a read of another and adds no wait between them;
  // the stage is a constant wherever this is called)
  static __device__ __forceinline__ uint8_t* stage(int st) {
    if constexpr (C::kTracked) {
      __shared__ __attribute__((aligned(16))) uint8_t s0[C::kStage];
      __shared__ __attribute__((aligned(16))) uint8_t s1[C::kStage];
      __shared__ __attribute__((aligned(16))) uint8_t s2[C::kStage];
      return st == 0 ? s0 : (st == 1 ? s1 : s2);
    } else {
      __shared__ __attribute__((aligned(16))) uint8_t v[C::kS * C::kStage];
      return v + st * C::kStage;
    }
  }
  static __device__ __forceinline__ uint8_t* m(int st) { return stage(st); }
  static __device__ __forceinline__ uint8_t* a(int st) { return m(st) + C::kM; }
  static __device__ __forceinline__ uint8_t* x(int st) { return a(st) + C::kA; }
  static __device__ __forceinline__ uint8_t* b(int st) { return a(st) + C::kA + C::kXI * 256; }
};

// MS = 32: the bf16 contraction runs on the 32x32x16 MFMA (on gfx950 the
// 16x16x32 bf16 shape issues at about half the rate of the 32x32 one).  A
// 32 x 32 block is a pair of 16-row sub-tiles by a pair of 16-column
// sub-tiles.  The packed fragments hold, for lane c + 16q of a sub-tile,
// column c and k = 32q .. 32q + 31; one permlane16 swap per code dword of a
// sub-tile pair hands each lane column c (lane bit 4 clear) or c + 16 (set)
// of the pair with k = 64h + 32R + 8s + (0..7) (h = lane / 32) in the
// swap's result R, dword s: the B operand of instruction (R, s).  The A
// operand reads the same k from the LDS tile.  Dense layers, bf16
// activations, INT and MXFP4 weights.
// Waves per SIMD a tile instance is held to (its register budget): the FP8
// 128 x 128 tile fits 128 VGPRs, which lets four workgroups share a CU (as
// many as its LDS admits); the others take what they need.
constexpr int tile_min_waves(int fmt, int wm, int wn, int amode, int epi, int s, int ms, bool sk) {
  return (fmt == F_FP8 && wm == 8 && wn == 2 && amode == A_DIRECT && epi == EPI_BF16 && s == 2 && ms == 16 && !sk) ? 4 : 1;
}

template <int FMT, int WM, int WN, int AMODE, int EPI, int S, int MS = 16, bool SK = false>
__global__ __launch_bounds__(256, tile_min_waves(FMT, WM, WN, AMODE, EPI, S, MS, SK)) void tile_kernel(const GemmParams p) {
  using C = TileCfg<FMT, WM, WN, AMODE, EPI, S>;
  using T = typename C::T;
  constexpr int kAE = T::kAElem;
  static_assert(MS == 16 || (MS == 32 && (fmt_int(FMT) || FMT == F_MXFP4_BF16) && WM % 2 == 0 && WN % 2 == 0 &&
                             AMODE == A_DIRECT && EPI == EPI_BF16),
                "32x32 blocks: dense bf16-activation INT / MXFP4 tiles of even sub-tile counts");
  static_assert(!SK || (AMODE == A_DIRECT && EPI == EPI_BF16), "Stream-K: dense tiles");
  constexpr int MP = MS == 32 ? WM / 2 : 1, NP = MS == 32 ? WN / 2 : 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wn = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, lg = lane >> 4;

  // XCD-aware order: consecutive workgroup ids go round-robin over the 8
  // XCDs; remap them so that each XCD walks a contiguous range of tiles.
  // Within it, tiles go in groups of group_m M-tiles by all N-tiles, M
  // fastest: the workgroups one XCD runs at a time then share both their
  // activation rows and their weight columns through that XCD's L2.  (MoE
  // launches take group_m = 1: N fastest over each expert block.)
  // Grouped rows with a live prefix: only the first `live` work items hold
  // rows, and a plain contiguous split would leave them on the first XCDs
  // (at 29 live expert blocks of 128 launched, two XCDs of eight), so each
  // XCD takes an equal contiguous share of the live items and its other
  // workgroups exit at once.  (The masked layout, whose live blocks lie at
  // the start of every expert's buffer, keeps the plain contiguous split:
  // the hardware's round-robin order spread each block's N-tiles over all
  // XCDs, each then fetching the block's rows, and ran 1.3-1.6x slower.)
  const uint32_t nwg = gridDim.x;
  uint32_t bid = blockIdx.x;
  uint32_t m_tiles = SK ? (uint32_t)p.sk_m_tiles : nwg / ((uint32_t)p.split_k * (uint32_t)p.n_tiles);
  uint32_t live = nwg;
  if constexpr (AMODE != A_DIRECT || EPI == EPI_SCATTER) {
    if (p.live_rows) {
      // the live M-tiles are the tile grid (groups of group_m over them)
      const int64_t rows = *p.live_rows;
      const int64_t lm = rows > 0 ? (rows + C::kTM - 1) / C::kTM : 0;
      if (lm < (int64_t)m_tiles) m_tiles = (uint32_t)lm;
      live = m_tiles * (uint32_t)p.n_tiles * (uint32_t)p.split_k;
    }
  }
  if (nwg % 8 == 0) {
    const uint32_t per = (live + 7) / 8, local = bid / 8;
    if (local >= per) return;
    bid = (bid % 8) * per + local;
  }
  if (bid >= live) return;
  // tile index -> (M-tile, N-tile)
  auto tile_coords = [&](uint32_t t, int64_t& tm, int& tn) {
    const uint32_t per_group = (uint32_t)p.group_m * (uint32_t)p.n_tiles;
    const uint32_t g = t / per_group, r = t % per_group;
    const uint32_t m0 = g * (uint32_t)p.group_m;
    const uint32_t gm = m_tiles - m0 < (uint32_t)p.group_m ? m_tiles - m0 : (uint32_t)p.group_m;
    tm = m0 + r % gm;
    tn = (int)(r / gm);
  };
  __shared__ int s_sk_last;

  // One tile's K-blocks [kb_begin, kb_end): the whole tile, a split-K share
  // (fp32 partials for the reduce kernel), or a Stream-K segment of tile
  // sk_tile (>= 0) taken by workgroup sk_g.
  auto tile_work = [&](int64_t tm, int tn, int split, int kb_begin, int kb_end, int sk_tile, int64_t sk_g) -> void {
  int expert = 0;
  if constexpr (AMODE != A_DIRECT || EPI == EPI_SCATTER) {  // grouped rows: the block's expert (-1: all padding)
    expert = p.block_expert[tm];
    if (expert < 0) return;
  }
  const int64_t row0 = tm * C::kTM;
  WPtrs wp;
  wp.codes = p.codes + (int64_t)expert * p.codes_per_expert;
  wp.meta = p.wscale + (int64_t)expert * p.scales_per_expert;
  // without zero points the (unused) zero words come from the scale array
  wp.zero = p.wzero ? p.wzero + (int64_t)expert * p.zeros_per_expert : wp.meta;
  const float gs = p.gscale[expert];

  int nts[WN];
  bool ntv[WN];
#pragma unroll
  for (int ns = 0; ns < WN; ++ns) {
    if constexpr (C::kSwiglu) {
      const int ntg = tn * (C::kTNS / 2) + wn * (WN / 2) + ns % (WN / 2);
      ntv[ns] = ntg * 16 < p.n;
      nts[ns] = ntg + (ns >= WN / 2 ? p.swiglu_nt_off : 0);
    } else {
      nts[ns] = tn * C::kTNS + wn * WN + ns;
      ntv[ns] = nts[ns] < p.nt_count;
    }
  }

  const int nkb = kb_end > kb_begin ? kb_end - kb_begin : 0;

  // --- DMA sources (every lane always gets a valid address: rows past the
  // end or padding read row 0 / slot 0, whose outputs are never stored) ---
  auto src_row = [&](int r) -> int64_t {
    const int64_t row = row0 + r;
    if (AMODE == A_GATHER) {
      const int32_t f = row < p.m ? p.sorted[row] : p.sentinel;
      return f < p.sentinel ? (int64_t)(f / p.topk) : 0;
    }
    return row < p.m ? row : 0;
  };
  // each buffer resource twice: as words for the inline-assembly copies and
  // as the builtin's type for the tracked ones
  const u32x4_t ra = rsrc_words(p.a, p.a_bytes);
  const __amdgpu_buffer_rsrc_t rar = make_rsrc(p.a, p.a_bytes);
  uint32_t a_off[C::kAIW];  // activation chunk of this lane in each of the wave's instructions (K-block 0)
  // (every wave issues kAIW instructions; with fewer than 4 in the tile,
  // waves repeat one -- same bytes to the same place -- so that the count of
  // DMAs in flight is the same on every path, which the compiler's waits
  // rely on)
#pragma unroll
  for (int i = 0; i < C::kAIW; ++i) {
    const int ins = (wn + 4 * i) % C::kAI;
    const int slot = ins * 64 + lane;
    const int r = slot / C::kCPR;
    const int lc = swz(r, slot % C::kCPR, C::kCPR, MS == 16);
    a_off[i] = (uint32_t)(src_row(r) * T::row_bytes(p.lda) + lc * 16);
  }
  u32x4_t rx = ra;
  __amdgpu_buffer_rsrc_t rxr = rar;
  uint32_t x_off[C::kXI > 0 ? C::kXI : 1];
  if constexpr (C::kX) {
    rx = rsrc_words(p.a_scale, p.a_scale_bytes);
    rxr = make_rsrc(p.a_scale, p.a_scale_bytes);
#pragma unroll
    for (int i = 0; i < C::kXI; ++i) {
      const int r = i * 64 + lane < C::kTM ? i * 64 + lane : 0;
      const int64_t sr = src_row(r);
      x_off[i] = (uint32_t)(sr * p.a_scale_ld);
    }
  }
  __amdgpu_buffer_rsrc_t rbr[WN];  // code stripes (invalid sub-tiles read sub-tile 0)
#pragma unroll
  for (int ns = 0; ns < WN; ++ns) {
    const int64_t cb = (int64_t)p.kb_count * C::kCB;
    const uint8_t* base = wp.codes + (ntv[ns] ? (int64_t)nts[ns] : 0) * cb;
    rbr[ns] = make_rsrc(base, cb);
  }
  // register-loaded fragments, one set per stage
  BFrag<FMT> bA[WN], bB[WN], bC[WN];
  // metadata words of the wave's sub-tiles.  INT: one copy per K-block, lane
  // l takes scale dword l / WN (of 8 for bf16 scales, 16 for f32) of
  // sub-tile l % WN, so that a lane finds its word of every sub-tile side by
  // side (one vector read).  (Zero points enter through the offset terms
  // after the K loop.)  MX: lane l its E8M0 word of each sub-tile.
  u32x4_t rms = ra;
  __amdgpu_buffer_rsrc_t rmsr = rar;
  const int sf = p.scale_f32;
  uint32_t mi_off = 0, mi_gmul = 0;
  if constexpr (fmt_int(FMT)) {
    rms = rsrc_words(wp.meta, p.scales_per_expert);
    rmsr = make_rsrc(wp.meta, p.scales_per_expert);
    const int nsw = (8 << sf) * WN;  // scale words (<= 64)
    const int ww = lane < nsw ? lane : 0;
    const int sub = ww % WN, d = ww / WN;
    const uint32_t nt = ntv[sub] ? (uint32_t)nts[sub] : 0u;
    mi_off = nt * p.ng * 16 * (2 << sf) + d * 4;
    mi_gmul = 16u * (2u << sf);
  } else if constexpr (fmt_mx_meta(FMT) || FMT == F_MXFP4_MXFP4) {
    rms = rsrc_words(wp.meta, p.scales_per_expert);
    rmsr = make_rsrc(wp.meta, p.scales_per_expert);
  } else if constexpr (FMT == F_FP8_BLOCK) {
    // lane l < WN copies the f32 block scale of sub-tile l (per K-block)
    rms = rsrc_words(wp.meta, p.scales_per_expert);
    rmsr = make_rsrc(wp.meta, p.scales_per_expert);
    uint32_t ntl = 0;
#pragma unroll
    for (int ns = 0; ns < WN; ++ns)
      if (lane == ns && ntv[ns]) ntl = (uint32_t)nts[ns];
    mi_off = ntl * (uint32_t)p.kb_count * 4u;
  }

  // copies of K-block kb into stage st (this wave's share) and its weight
  // fragments into registers bdst
  using St = TileLds<FMT, WM, WN, AMODE, EPI, S>;
  // LDS DMA: inline assembly (untracked) or the builtin (tracked)
  using LdsPtr = __attribute__((address_space(3))) void*;
  auto dma16 = [&](const u32x4_t& rw, __amdgpu_buffer_rsrc_t rr, uint8_t* lds, uint32_t voff) -> void {
    if constexpr (C::kTracked)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (LdsPtr)lds, 16, voff, 0, 0, 0);
    else
      dma_b128(rw, lds, voff);
  };
  auto dma4 = [&](const u32x4_t& rw, __amdgpu_buffer_rsrc_t rr, uint8_t* lds, uint32_t voff) -> void {
    if constexpr (C::kTracked)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (LdsPtr)lds, 4, voff, 0, 0, 0);
    else
      dma_b32(rw, lds, voff);
  };
  auto issue = [&](int kb, int st, BFrag<FMT>* bdst) -> void {
#pragma unroll
    for (int i = 0; i < C::kAIW; ++i) {
      const int ins = (wn + 4 * i) % C::kAI;
      dma16(ra, rar, St::a(st) + ins * 1024, a_off[i] + (uint32_t)kb * C::kRowB);
    }
    // per-row words: every wave copies them all (same bytes, same place)
    if constexpr (C::kX) {
#pragma unroll
      for (int i = 0; i < C::kXI; ++i)
        dma4(rx, rxr, St::x(st) + i * 256, x_off[i] + (uint32_t)kb * 4);
    }
    {
      // (compiler-tracked loads.  A lane's kBWords 16-byte words sit side
      // by side in the packed layout.)
      const uint32_t boff = (uint32_t)kb * C::kCB + lane * T::kCodeB;
#pragma unroll
      for (int ns = 0; ns < WN; ++ns)
#pragma unroll
        for (int h = 0; h < T::kBWords; ++h)
          bdst[ns].w[h] = load_code_word<FMT>(rbr[ns], boff + h * 16);
      // (the offset stays live past the loads: no load's destination
      // reuses the register another load reads its address from)
      asm volatile("" ::"v"(boff));
    }
    uint8_t* mw = St::m(st) + wn * C::kMI * 256;
    if constexpr (fmt_int(FMT)) {
      const int gi = (int)(((float)kb + 0.5f) * p.inv_kbg);
      dma4(rms, rmsr, mw, mi_off + (uint32_t)gi * mi_gmul);
    } else if constexpr (FMT == F_FP8_BLOCK) {
      dma4(rms, rmsr, mw, mi_off + (uint32_t)kb * 4u);
    } else if constexpr (fmt_mx_meta(FMT) || FMT == F_MXFP4_MXFP4) {
      // a metadata row covers 4 K-blocks (E8M0 per 32) or 2 (NVFP4: two
      // E4M3 per 32 of a lane)
      constexpr int kRowShift = FMT == F_NVFP4_BF16 ? 1 : 2;
#pragma unroll
      for (int ns = 0; ns < WN; ++ns) {
        dma4(rms, rmsr, mw + ns * 256,
             ((uint32_t)((ntv[ns] ? nts[ns] : 0) * p.kb4 + (kb >> kRowShift)) * 64 + lane) * 4);
      }
    }
    // keep the issue ahead of the compute (the waits count on it)
    __builtin_amdgcn_sched_barrier(0);
  };
  // this wave's copies into the next stage have landed, so that after the
  // barrier every wave may read them.  Vector-memory loads complete in
  // order; with three stages the wave has issued since then only the kIss
  // loads of the stage after (the loop holds no other vector-memory
  // access), which stay in flight; with two, everything is waited for.
  // The compiler's own waits cover only this wave's reads of its own
  // copies, hence this one.
  constexpr int kIss = C::kAIW + C::kXI + WN * T::kBWords + C::kMI;
  static_assert(kIss < 64, "vmcnt range");
  constexpr int kAhead = C::kS == 3 ? kIss : 0;  // loads left in flight after the wait
  auto wait_own = [&]() -> void {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((kAhead & 15) | ((kAhead >> 4) << 14) | (7 << 4) | (15 << 8));
    __builtin_amdgcn_sched_barrier(0);
  };
  // workgroup barrier without a memory fence (the fence of __syncthreads()
  // would wait for every DMA in flight, prefetches included); the empty asm
  // keeps the compiler from moving memory accesses across it
  auto barrier = [&]() -> void {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
  };

  f32x4_t acc[WM][WN];
#pragma unroll
  for (int ms = 0; ms < WM; ++ms)
#pragma unroll
    for (int ns = 0; ns < WN; ++ns) acc[ms][ns] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // (MS = 32) 32 x 32 accumulators in the MFMA's C layout: register i of
  // lane l holds row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32
  f32x16_t acc32[MP][NP];
#pragma unroll
  for (int mp = 0; mp < MP; ++mp)
#pragma unroll
    for (int np = 0; np < NP; ++np)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc32[mp][np][i] = 0.0f;

  const IntScaleSel ssel = int_scale_sel(p, c16);
  auto compute = [&](int kb, int st, const BFrag<FMT>* bsrc) -> void {
    const uint8_t* abase = St::a(st);
    const uint8_t* bbase = St::b(st) + wn * WN * C::kCB;
    const uint8_t* mbase = St::m(st) + wn * C::kMI * 256;
    BFrag<FMT> bf[WN];
    uint32_t mw[WN];
#pragma unroll
    for (int ns = 0; ns < WN; ++ns) {
#pragma unroll
      for (int h = 0; h < T::kBWords; ++h)
        bf[ns].w[h] = C::kBReg ? bsrc[ns].w[h]
                               : *reinterpret_cast<const CodeW<FMT>*>(bbase + ns * C::kCB + lane * T::kCodeB + h * 16);
      mw[ns] = 0;
      if constexpr (fmt_mx_meta(FMT) || FMT == F_MXFP4_MXFP4)
        mw[ns] = *reinterpret_cast<const uint32_t*>(mbase + ns * 256 + lane * 4);
    }
    if constexpr (FMT == F_FP8_BLOCK) {
      // the WN block scales of this K-block, side by side
      struct alignas(4 * WN) Words { float w[WN]; };
      const Words sw = *reinterpret_cast<const Words*>(mbase);
#pragma unroll
      for (int ms = 0; ms < WM; ++ms) {
        const int r = ms * 16 + c16;
        const int swr = (r >> 1) & 7;
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(abase + r * C::kRowB + ((lg ^ swr) * 16));
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(abase + r * C::kRowB + (((4 + lg) ^ swr) * 16));
        i32x8_t a8;
        a8[0] = lo[0]; a8[1] = lo[1]; a8[2] = lo[2]; a8[3] = lo[3];
        a8[4] = hi[0]; a8[5] = hi[1]; a8[6] = hi[2]; a8[7] = hi[3];
        // the f32 group scales of this lane's 4 output rows (C layout)
        const f32x4_t sa = *reinterpret_cast<const f32x4_t*>(St::x(st) + (ms * 16 + 4 * lg) * 4);
#pragma unroll
        for (int ns = 0; ns < WN; ++ns) {
          const f32x4_t t = mfma_f8_kblock<FMT>(a8, 127, bf[ns], 0u, kb, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[ms][ns][i] = __builtin_fmaf(sa[i] * sw.w[ns], t[i], acc[ms][ns][i]);
        }
      }
      return;
    }
    if constexpr (fmt_int(FMT)) {
      // this lane's scale words of the WN sub-tiles, side by side (one
      // aligned vector read)
      struct alignas(4 * WN) Words { uint32_t w[WN]; };
      const Words sw = *reinterpret_cast<const Words*>(mbase + (sf ? c16 : (c16 >> 1)) * WN * 4);
#pragma unroll
      for (int ns = 0; ns < WN; ++ns) mw[ns] = sw.w[ns];
    }
    if constexpr (T::kBf16 && MS == 32) {
      const int h = lane >> 5;
      const bool hi = (lane & 16) != 0;  // the lane's column is in the pair's second sub-tile
      // code dwords after the swap, [pair][R][dword] (a lane's 4-bit codes:
      // dword s = step s; b-bit integers: their b bit-plane dwords)
      constexpr int kND = T::kCodeB / 4;
      CodeW<FMT> cw[NP][2];
      uint32_t mp2[NP][2];    // MXFP4: E8M0 words after the same swap
#pragma unroll
      for (int np = 0; np < NP; ++np) {
#pragma unroll
        for (int s = 0; s < kND; ++s) {
          const auto r = __builtin_amdgcn_permlane16_swap(bf[2 * np].w[0][s], bf[2 * np + 1].w[0][s], false, false);
          cw[np][0][s] = r[0];
          cw[np][1][s] = r[1];
        }
        if constexpr (FMT == F_MXFP4_BF16) {
          const auto r = __builtin_amdgcn_permlane16_swap(mw[2 * np], mw[2 * np + 1], false, false);
          mp2[np][0] = r[0];
          mp2[np][1] = r[1];
        }
      }
      // INT: one K-block of (128 + u) codes into fresh accumulators, then
      // scaled by the lane's column scale (the offset is taken off after the
      // K loop); MXFP4: scaled in the widening, accumulated in place
      f32x16_t tk[MP][NP];
      if constexpr (fmt_int(FMT)) {
#pragma unroll
        for (int mp = 0; mp < MP; ++mp)
#pragma unroll
          for (int np = 0; np < NP; ++np)
#pragma unroll
            for (int i = 0; i < 16; ++i) tk[mp][np][i] = 0.0f;
      }
#pragma unroll
      for (int R = 0; R < 2; ++R)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          bf16x8_t dd[NP];
#pragma unroll
          for (int np = 0; np < NP; ++np) {
            if constexpr (fmt_int(FMT))
              dd[np] = int_dequant_step<T::kIntBits>(cw[np][R], s);
            else
              dd[np] = mx_dequant(cw[np][R][s], e8m0_to_f32(frag_mx_code(mp2[np][R], kb)));
          }
#pragma unroll
          for (int mp = 0; mp < MP; ++mp) {
            const int r = mp * 32 + (lane & 31);
            const int chunk = 8 * h + 4 * R + s;
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(abase + r * C::kRowB + ((chunk ^ (r & 15)) * 16));
#pragma unroll
            for (int np = 0; np < NP; ++np) {
              if constexpr (fmt_int(FMT))
                tk[mp][np] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dd[np], tk[mp][np], 0, 0, 0);
              else
                acc32[mp][np] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dd[np], acc32[mp][np], 0, 0, 0);
            }
          }
        }
      if constexpr (fmt_int(FMT)) {
#pragma unroll
        for (int np = 0; np < NP; ++np) {
          // the scale word of the lane's column (sub-tile 2 np + hi), read
          // from LDS by address (a per-lane choice between two elements of
          // a register array would be turned into an indexed array access)
          const uint32_t mwl = *reinterpret_cast<const uint32_t*>(mbase + (sf ? c16 : (c16 >> 1)) * WN * 4 +
                                                                   (2 * np + (hi ? 1 : 0)) * 4);
          const float sc = frag_int_scale(mwl, ssel);
#pragma unroll
          for (int mp = 0; mp < MP; ++mp)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc32[mp][np][i] = __builtin_fmaf(sc, tk[mp][np][i], acc32[mp][np][i]);
        }
      }
    } else if constexpr (T::kBf16) {
      bf16x8_t d[WN][4];
#pragma unroll
      for (int ns = 0; ns < WN; ++ns) dequant_b<FMT>(bf[ns], mw[ns], kb, d[ns]);
#pragma unroll
      for (int ms = 0; ms < WM; ++ms) {
        const int r = ms * 16 + c16;
        bf16x8_t af[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
          af[s] = *reinterpret_cast<const bf16x8_t*>(abase + r * C::kRowB + (swz(r, 4 * lg + s, 16, true) * 16));
        if constexpr (fmt_int(FMT)) {
          // one K-block of (128 + u) codes, scaled; the offset it carries
          // is taken off after the K loop
#pragma unroll
          for (int ns = 0; ns < WN; ++ns) {
            const f32x4_t t = mfma_bf16_kblock(af, d[ns], f32x4_t{0.0f, 0.0f, 0.0f, 0.0f});
            const float sc = frag_int_scale(mw[ns], ssel);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[ms][ns][i] = __builtin_fmaf(sc, t[i], acc[ms][ns][i]);
          }
        } else {
#pragma unroll
          for (int ns = 0; ns < WN; ++ns) acc[ms][ns] = mfma_bf16_kblock(af, d[ns], acc[ms][ns]);
        }
      }
    } else {
#pragma unroll
      for (int ms = 0; ms < WM; ++ms) {
        const int r = ms * 16 + c16;
        i32x8_t a8;
        if constexpr (T::kA4) {
          // 32 E2M1 codes of k = 32 lg + j: one 16-byte chunk
          const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(abase + r * C::kRowB + (swz(r, lg, 4) * 16));
          a8[0] = lo[0]; a8[1] = lo[1]; a8[2] = lo[2]; a8[3] = lo[3];
          a8[4] = 0; a8[5] = 0; a8[6] = 0; a8[7] = 0;
        } else {
          const int sw = (r >> 1) & 7;
          const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(abase + r * C::kRowB + ((lg ^ sw) * 16));
          const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(abase + r * C::kRowB + (((4 + lg) ^ sw) * 16));
          a8[0] = lo[0]; a8[1] = lo[1]; a8[2] = lo[2]; a8[3] = lo[3];
          a8[4] = hi[0]; a8[5] = hi[1]; a8[6] = hi[2]; a8[7] = hi[3];
        }
        int sa = 127;
        if (C::kX) sa = (int)((reinterpret_cast<const uint32_t*>(St::x(st))[r] >> (8 * lg)) & 0xFF);
#pragma unroll
        for (int ns = 0; ns < WN; ++ns) acc[ms][ns] = mfma_f8_kblock<FMT>(a8, sa, bf[ns], mw[ns], kb, acc[ms][ns]);
      }
    }
  };

  if (nkb > 0) {
    // K-block j uses stage j % kS and register set j % kS.  In the loop the
    // copies are issued unconditionally (past the last K-block they re-read
    // that block into a stage that is never consumed): the count of loads in
    // flight is then the same on every path, which the explicit waits rely
    // on.  The loop is unrolled kS times, so that every stage and register
    // set is a constant and the accumulators stay in the same registers.
    const int kb_last = kb_begin + nkb - 1;
    auto kb_at = [&](int j) -> int { return kb_begin + j <= kb_last ? kb_begin + j : kb_last; };
    if constexpr (C::kS == 2) {
      issue(kb_at(0), 0, bA);
      wait_own();
      barrier();
      int j = 0;
      for (; j + 1 < nkb; j += 2) {
        issue(kb_at(j + 1), 1, bB);
        compute(kb_begin + j, 0, bA);
        wait_own();
        barrier();
        issue(kb_at(j + 2), 0, bA);
        compute(kb_begin + j + 1, 1, bB);
        wait_own();
        barrier();
      }
      if (j < nkb) compute(kb_begin + j, 0, bA);
    } else {
      issue(kb_at(0), 0, bA);
      issue(kb_at(1), 1, bB);
      wait_own();
      barrier();
      int j = 0;
      for (; j + 2 < nkb; j += 3) {
        issue(kb_at(j + 2), 2, bC);
        compute(kb_begin + j, 0, bA);
        wait_own();
        barrier();
        issue(kb_at(j + 3), 0, bA);
        compute(kb_begin + j + 1, 1, bB);
        wait_own();
        barrier();
        issue(kb_at(j + 4), 1, bB);
        compute(kb_begin + j + 2, 2, bC);
        wait_own();
        barrier();
      }
      // one or two K-blocks left, their copies issued: nothing more to
      // issue, so wait for everything
      if (j < nkb) {
        compute(kb_begin + j, 0, bA);
        if (j + 1 < nkb) {
          __builtin_amdgcn_s_waitcnt(0);
          barrier();
          compute(kb_begin + j + 1, 1, bB);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no DMA outlives the workgroup's LDS

  if constexpr (fmt_int(FMT)) {
    // The K loop summed s * (128 + u) a per K-block; the offset part,
    // sum over K-blocks of s (offset + z) * (sum of the block's a), is one
    // more small product, taken here on the MFMA: row sums (A) times the
    // weight's offset terms (B, stored negated) with K running over
    // K-blocks, each operand as a bf16 hi / lo pair (hi*hi + hi*lo + lo*hi).
    // The share that starts at K-block 0 adds the whole of it.
    if (kb_begin == 0 && MS == 32) {
      // the same product on the 32x32x16 MFMA: row sums of a pair of 16-row
      // tiles and offset terms of a pair of sub-tiles, each swapped into the
      // 32-wide operand layout as the weight codes are (K-block slots
      // 8 lg + (0..7) of the 16-wide layouts: lane groups 0 / 2 in the
      // swap's result 0, 1 / 3 in result 1)
      const int64_t mt16 = (p.m + 15) / 16;
      const int64_t rs_half = mt16 * p.kbc * 1024;
      const int64_t co_half = (int64_t)p.nt_count * p.kbc * 1024;
      const uint8_t* cob = p.wco + (int64_t)expert * p.co_per_expert;
      auto swap4 = [](const u32x4_t& x, const u32x4_t& y, u32x4_t& r0, u32x4_t& r1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const auto r = __builtin_amdgcn_permlane16_swap(x[j], y[j], false, false);
          r0[j] = r[0];
          r1[j] = r[1];
        }
      };
      for (int cc = 0; cc < p.kbc; ++cc) {
        u32x4_t ch[NP][2], cl[NP][2];
#pragma unroll
        for (int np = 0; np < NP; ++np) {
          u32x4_t xh[2], xl[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int ns = 2 * np + q;
            const int64_t o = (((int64_t)(ntv[ns] ? nts[ns] : 0) * p.kbc + cc) * 64 + lane) * 16;
            xh[q] = *reinterpret_cast<const u32x4_t*>(cob + o);
            xl[q] = *reinterpret_cast<const u32x4_t*>(cob + co_half + o);
          }
          swap4(xh[0], xh[1], ch[np][0], ch[np][1]);
          swap4(xl[0], xl[1], cl[np][0], cl[np][1]);
        }
#pragma unroll
        for (int mp = 0; mp < MP; ++mp) {
          u32x4_t yh[2], yl[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int64_t mt = row0 / 16 + 2 * mp + q;
            // (16-row tiles past m have no row sums: zero, their rows are never stored)
            const int64_t o = ((mt * p.kbc + cc) * 64 + lane) * 16;
            yh[q] = mt < mt16 ? *reinterpret_cast<const u32x4_t*>(p.a_rowsum + o) : u32x4_t{0, 0, 0, 0};
            yl[q] = mt < mt16 ? *reinterpret_cast<const u32x4_t*>(p.a_rowsum + rs_half + o) : u32x4_t{0, 0, 0, 0};
          }
          u32x4_t rh[2], rl[2];
          swap4(yh[0], yh[1], rh[0], rh[1]);
          swap4(yl[0], yl[1], rl[0], rl[1]);
#pragma unroll
          for (int R = 0; R < 2; ++R) {
            const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, rh[R]), al = __builtin_bit_cast(bf16x8_t, rl[R]);
#pragma unroll
            for (int np = 0; np < NP; ++np) {
              const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, ch[np][R]), bl = __builtin_bit_cast(bf16x8_t, cl[np][R]);
              acc32[mp][np] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc32[mp][np], 0, 0, 0);
              acc32[mp][np] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc32[mp][np], 0, 0, 0);
              acc32[mp][np] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc32[mp][np], 0, 0, 0);
            }
          }
        }
      }
    } else if (kb_begin == 0) {
      const int64_t mt16 = (p.m + 15) / 16;
      const int64_t rs_half = mt16 * p.kbc * 1024;
      const int64_t co_half = (int64_t)p.nt_count * p.kbc * 1024;
      const uint8_t* cob = p.wco + (int64_t)expert * p.co_per_expert;
      for (int cc = 0; cc < p.kbc; ++cc) {
        bf16x8_t ch[WN], cl[WN];
#pragma unroll
        for (int ns = 0; ns < WN; ++ns) {
          const int64_t o = (((int64_t)(ntv[ns] ? nts[ns] : 0) * p.kbc + cc) * 64 + lane) * 16;
          ch[ns] = *reinterpret_cast<const bf16x8_t*>(cob + o);
          cl[ns] = *reinterpret_cast<const bf16x8_t*>(cob + co_half + o);
        }
#pragma unroll
        for (int ms = 0; ms < WM; ++ms) {
          const int64_t mt = row0 / 16 + ms;
          if (mt >= mt16) break;  // rows past m: never stored
          const int64_t o = ((mt * p.kbc + cc) * 64 + lane) * 16;
          const bf16x8_t rh = *reinterpret_cast<const bf16x8_t*>(p.a_rowsum + o);
          const bf16x8_t rl = *reinterpret_cast<const bf16x8_t*>(p.a_rowsum + rs_half + o);
#pragma unroll
          for (int ns = 0; ns < WN; ++ns) {
            acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rh, ch[ns], acc[ms][ns], 0, 0, 0);
            acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rh, cl[ns], acc[ms][ns], 0, 0, 0);
            acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rl, ch[ns], acc[ms][ns], 0, 0, 0);
          }
        }
      }
    }
  }

  if constexpr (SK) {
    // Stream-K: workgroup g takes iterations [g L, (g + 1) L) of the tiles'
    // K-blocks laid end to end, so a tile's K-blocks may be shared by the
    // workgroups g_first .. g_last.  Each of them writes its partial sums
    // (slot 2 g for the first tile of its range, 2 g + 1 for the last); the
    // last to finish adds every segment's slot in segment order -- a fixed
    // order, so the result does not depend on which one finishes last --
    // and stores the tile.  The counter is left at zero for the next call.
    const int64_t KB = p.kb_count, L = p.sk_len;
    const int64_t g_first = ((int64_t)sk_tile * KB) / L;
    const int64_t g_last = ((int64_t)sk_tile * KB + KB - 1) / L;
    const int nseg = (int)(g_last - g_first + 1);
    if (nseg > 1) {
      constexpr int kV = WM * WN;  // f32x4 of accumulators per lane
      // The slots are written and read with device-coherent accesses (the
      // cache policy of a device-scope atomic access: through to memory,
      // around the XCD's L2), so no fence has to write back or invalidate a
      // whole L2 -- which would cost every workgroup on that XCD its cached
      // operands.
      constexpr int kDev = 16;  // sc1
      const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.sk_part, p.sk_part_bytes);
      auto slot = [&](int64_t g) -> uint32_t {
        const int64_t sl = 2 * g + (((g * L) / KB) == sk_tile ? 0 : 1);
        return (uint32_t)((((sl * 4 + wn) * kV) * 64 + lane) * 16);
      };
      auto acc_at = [&](int v) -> f32x4_t& {
        if constexpr (MS == 32) {
          // (f32x16 accumulators as four f32x4 each)
          return reinterpret_cast<f32x4_t*>(&acc32[v / (4 * NP)][(v / 4) % NP])[v % 4];
        } else {
          return acc[v / WN][v % WN];
        }
      };
      const uint32_t mine = slot(sk_g);
#pragma unroll
      for (int v = 0; v < kV; ++v)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc_at(v)), rp, mine + v * 1024, 0, kDev);
      // every wave's slot stores have completed before the count goes up
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(p.sk_count + sk_tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old + 1 == (uint32_t)nseg;
        if (last) __hip_atomic_store(p.sk_count + sk_tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_sk_last = last;
      }
      __syncthreads();
      if (!s_sk_last) return;
      for (int i = 0; i < nseg; ++i) {
        const uint32_t src = slot(g_first + i);
#pragma unroll
        for (int v = 0; v < kV; ++v) {
          const f32x4_t x = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, src + v * 1024, 0, kDev));
          acc_at(v) = i == 0 ? x : acc_at(v) + x;
        }
      }
    }
  }

  if constexpr (MS == 32) {
    // 32 x 32 blocks: lane l holds column l % 32 of its pair and rows
    // 8 (i / 4) + 4 (l / 32) + i % 4
    const int64_t ncols = (int64_t)p.nt_count * 16;
    const int h = lane >> 5;
#pragma unroll
    for (int np = 0; np < NP; ++np) {
      // the pair's sub-tiles are consecutive: column nts[2 np] * 16 + l % 32
      // (past N: never stored)
      const int64_t col = (int64_t)nts[2 * np] * 16 + (lane & 31);
      if (col >= p.n) continue;
      const float cs = col_scale<FMT>(wp.meta, col, gs);
      const float bias = p.bias ? bf16_bits_to_f32(p.bias[col]) : 0.0f;
#pragma unroll
      for (int mp = 0; mp < MP; ++mp) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t row = row0 + 32 * mp + 8 * (i >> 2) + 4 * h + (i & 3);
          if (row >= p.m) continue;
          if (p.split_k > 1) {
            p.partials[((int64_t)split * p.m + row) * ncols + col] = acc32[mp][np][i];
          } else {
            uint16_t* out = static_cast<uint16_t*>(p.out);
            out[row * p.ldo + col] = (uint16_t)f32_to_bf16_bits(acc32[mp][np][i] * cs + bias);
          }
        }
      }
    }
    return;
  }
  if (p.split_k > 1) {
    const int64_t ncols = C::kSwiglu ? 2 * p.n : (int64_t)p.nt_count * 16;
#pragma unroll
    for (int ns = 0; ns < WN; ++ns) {
      if (!ntv[ns]) continue;
#pragma unroll
      for (int ms = 0; ms < WM; ++ms)
        store_partial(p, split, row0 + ms * 16, (int64_t)nts[ns] * 16 + c16, ncols, acc[ms][ns], lg);
    }
    return;
  }
  if constexpr (MS == 16 && (EPI == EPI_SCATTER || (EPI == EPI_BF16 && AMODE == A_DIRECT))) {
    // Output through LDS: in the 16x16 C layout a lane holds four rows of
    // one column, so direct stores are 2 bytes wide (and, for the MoE down
    // GEMM, to rows scattered over the output).  Instead the tile goes out
    // in slices of rows: each lane writes its bf16 values of those rows into
    // a row-major staging area (the pipeline's first stage, free after the K
    // loop), and every thread then stores 16 contiguous bytes of one row to
    // its output row (its flat slot for the scatter).  Measured on MI355X:
    // the MoE W4A8 layer at T = 8192 went from 1489 to 1308 us with 8-row
    // slices, then to about 1120 with the slots loaded up front, 16-row
    // slices and LDS-only barriers; dense FP8 W8A8 at M = 4096, N = 7168, K =
    // 2048 from 98 to 88 us.
    constexpr int kCols = C::kTNS * 16;           // columns of the workgroup tile
    constexpr int kChunks = kCols / 8;            // 16-byte chunks per row
    constexpr int kRowB = kCols * 2;
    // rows per slice (a whole 16-row block where a stage holds it, so that
    // every lane converts and writes in every slice; else 8 or 4) and the
    // staged row pitch (padded by 16 bytes where room allows: rows 4 apart
    // then fall on other banks)
    constexpr int kSlice = (16 * kRowB <= C::kStage) ? 16 : ((8 * kRowB <= C::kStage) ? 8 : 4);
    constexpr int kPitch = kRowB + ((kSlice * (kRowB + 16) <= C::kStage) ? 16 : 0);
    static_assert(kSlice * kPitch <= C::kStage, "staged output rows fit one pipeline stage");
    uint8_t* ep = St::stage(0);
    uint16_t* out = static_cast<uint16_t*>(p.out);
    const int64_t col_base = (int64_t)tn * kCols;
    // 16-byte stores need 16-byte aligned rows; else 2-byte stores from LDS
    const bool vec = (p.ldo % 8) == 0 && ((uintptr_t)p.out & 15) == 0;
    // The flat slots of the rows this thread stores, every slice's loaded at
    // once and only compared at their use: one memory latency for the
    // epilogue rather than one per slice (each slice ends in a barrier, so
    // loads issued inside it would wait in turn).  Rows past m load row0's
    // slot (the block is live, so row0 < m) and are skipped by `in`.
    constexpr int kSlices = (16 / kSlice) * WM;
    constexpr int kPer = (kSlice * kChunks + 255) / 256;
    int32_t slot[kSlices][kPer];
    bool in[kSlices][kPer];
#pragma unroll
    for (int pz = 0; pz < kSlices; ++pz) {
      const int ms = pz / (16 / kSlice), h = pz % (16 / kSlice);
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int sidx = tid + 256 * q;
        const int64_t row = row0 + ms * 16 + kSlice * h + sidx / kChunks;
        in[pz][q] = sidx < kSlice * kChunks && row < p.m;
        if constexpr (EPI == EPI_SCATTER)
          slot[pz][q] = p.sorted[in[pz][q] ? row : row0];
        else
          slot[pz][q] = (int32_t)row;  // dense rows: the output row itself
      }
    }
    // column scales (read after the K loop: loaded any earlier they would
    // hold registers through it)
    float cs[WN], bias[WN];
#pragma unroll
    for (int ns = 0; ns < WN; ++ns) {
      const int64_t col = (int64_t)nts[ns] * 16 + c16;
      const bool cv = col < p.n;
      cs[ns] = cv ? col_scale<FMT>(wp.meta, col, gs) : 0.0f;
      bias[ns] = (EPI == EPI_BF16 && p.bias && cv) ? bf16_bits_to_f32(p.bias[col]) : 0.0f;
    }
    // a barrier for the staging area alone: this wave's LDS accesses done,
    // its stores to the output left in flight
    auto lds_barrier = [&]() -> void {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
    };
#pragma unroll
    for (int pz = 0; pz < kSlices; ++pz) {
      const int ms = pz / (16 / kSlice), h = pz % (16 / kSlice);
      // every wave is past its reads of the stage (the last K-block's
      // operands, or the previous slice).  The first time with a full wait:
      // the pipeline's trailing copies (and the slot loads) land first.
      if (pz == 0)
        __syncthreads();
      else
        lds_barrier();
      if ((4 * lg) / kSlice == h) {
        // rows in pairs: one conversion instruction per two values
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const int r8 = 4 * lg + i - kSlice * h;  // row within the slice
          float rs0 = 1.0f, rs1 = 1.0f;
          if constexpr (FMT == F_FP8) {
            const int64_t row = row0 + ms * 16 + 4 * lg + i;
            rs0 = row < p.m ? row_act_scale<FMT, AMODE>(p, row) : 1.0f;
            rs1 = row + 1 < p.m ? row_act_scale<FMT, AMODE>(p, row + 1) : 1.0f;
          }
#pragma unroll
          for (int ns = 0; ns < WN; ++ns) {
            const uint32_t pr = f32x2_to_bf16x2_bits(acc[ms][ns][i] * cs[ns] * rs0 + bias[ns],
                                                     acc[ms][ns][i + 1] * cs[ns] * rs1 + bias[ns]);
            uint8_t* e0 = ep + r8 * kPitch + ((wn * WN + ns) * 16 + c16) * 2;
            *reinterpret_cast<uint16_t*>(e0) = (uint16_t)pr;
            *reinterpret_cast<uint16_t*>(e0 + kPitch) = (uint16_t)(pr >> 16);
          }
        }
      }
      lds_barrier();
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int sidx = tid + 256 * q;
        if (!in[pz][q] || (EPI == EPI_SCATTER && slot[pz][q] >= p.sentinel)) continue;
        const int r8 = sidx / kChunks, ch = sidx % kChunks;
        const int64_t dst = slot[pz][q];
        const int64_t col0 = col_base + ch * 8;
        if (col0 >= p.n) continue;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ep + r8 * kPitch + ch * 16);
        if (vec && col0 + 8 <= p.n) {
          *reinterpret_cast<u32x4_t*>(out + dst * p.ldo + col0) = v;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (col0 + j < p.n) out[dst * p.ldo + col0 + j] = (uint16_t)(v[j >> 1] >> (16 * (j & 1)));
        }
      }
    }
    return;
  }
#pragma unroll
  for (int ms = 0; ms < WM; ++ms) {
    const int64_t rb = row0 + ms * 16;
    if constexpr (EPI == EPI_BF16 || EPI == EPI_SCATTER) {
#pragma unroll
      for (int ns = 0; ns < WN; ++ns) store_tile<FMT, EPI, AMODE>(p, wp.meta, gs, rb, (int64_t)nts[ns] * 16 + c16, acc[ms][ns], lg);
    } else if constexpr (EPI == EPI_SWIGLU_BF16) {
#pragma unroll
      for (int j = 0; j < WN / 2; ++j)
        store_swiglu_bf16<FMT, AMODE>(p, wp.meta, gs, rb, (int64_t)nts[j] * 16 + c16, acc[ms][j], acc[ms][j + WN / 2], lg);
    } else if constexpr (EPI == EPI_SWIGLU_MXFP4) {
#pragma unroll
      for (int jj = 0; jj < WN / 4; ++jj)
        store_swiglu_mxfp4<FMT>(p, wp.meta, gs, rb, (int64_t)nts[2 * jj] * 16 + c16, acc[ms][2 * jj], acc[ms][2 * jj + WN / 2],
                           acc[ms][2 * jj + 1], acc[ms][2 * jj + 1 + WN / 2], lg, c16);
    } else {
#pragma unroll
      for (int jj = 0; jj < WN / 4; ++jj)
        store_swiglu_mxfp8<FMT>(p, wp.meta, gs, rb, (int64_t)nts[2 * jj] * 16 + c16, acc[ms][2 * jj], acc[ms][2 * jj + WN / 2],
                           acc[ms][2 * jj + 1], acc[ms][2 * jj + 1 + WN / 2], lg, c16);
    }
  }
  };

  if constexpr (SK) {
    // Stream-K (dense layers): this workgroup's iterations [bid L, (bid + 1)
    // L) of the tiles' K-blocks laid end to end, one segment per tile they
    // touch
    const int64_t KB = p.kb_count, L = p.sk_len;
    const int64_t it_all = (int64_t)p.sk_tiles * KB;
    int64_t it = (int64_t)bid * L;
    const int64_t it_end = it + L < it_all ? it + L : it_all;
    bool first = true;
    while (it < it_end) {
      const int64_t t = it / KB;
      const int k0 = (int)(it - t * KB);
      const int k1 = (int)(it_end - it < KB - k0 ? k0 + (it_end - it) : KB);
      if (!first) __syncthreads();  // the previous segment's LDS reads are done
      int64_t tm;
      int tn;
      tile_coords((uint32_t)t, tm, tn);
      tile_work(tm, tn, 0, k0, k1, (int)t, (int64_t)bid);
      first = false;
      it += k1 - k0;
    }
  } else {
    const int split = (int)(bid % (uint32_t)p.split_k);
    int64_t tm;
    int tn;
    tile_coords(bid / (uint32_t)p.split_k, tm, tn);
    const int kb_begin = split * p.kb_per_split;
    int kb_end = kb_begin + p.kb_per_split;
    if (kb_end > p.kb_count) kb_end = p.kb_count;
    tile_work(tm, tn, split, kb_begin, kb_end, -1, 0);
  }
}

// ---------------------------------------------------------------------------
// Split-K reduce + epilogue: one thread per (row, 32-column block) for the
// MXFP8 epilogue, per (row, 8 columns) otherwise.  Partials are summed in
// split order.

template <int FMT, int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const GemmParams p, int block_m) {
  static_assert(EPI != EPI_SWIGLU_MXFP4, "no split-K for the MXFP4 SwiGLU epilogue");
  constexpr bool kSwiglu = (EPI == EPI_SWIGLU_BF16 || EPI == EPI_SWIGLU_MXFP8 || EPI == EPI_SWIGLU_MXFP4);
  constexpr int kCols = (EPI == EPI_SWIGLU_MXFP8) ? 32 : 8;
  const int64_t ncols = kSwiglu ? 2 * p.n : (int64_t)p.nt_count * 16;
  const int64_t outc = p.n;
  const int64_t cpr = (outc + kCols - 1) / kCols;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= p.m * cpr) return;
  const int64_t row = id / cpr;
  const int64_t c0 = (id % cpr) * kCols;
  int expert = 0;
  if (p.sorted) {
    if (p.sorted[row] >= p.sentinel) return;
    expert = p.block_expert[row / block_m];
  }
  const float gs = p.gscale[expert];
  const uint8_t* wmeta = p.wscale + (int64_t)expert * p.scales_per_expert;
  float v[kCols], u[kCols];
#pragma unroll
  for (int i = 0; i < kCols; ++i) v[i] = u[i] = 0.0f;
  // The loads are unconditional (columns past the end re-read the last
  // column, whose sums are never stored): a branch around each load would
  // make the compiler wait for it before the next one.  Four splits' loads
  // go out together.
  int cc[kCols];
#pragma unroll
  for (int i = 0; i < kCols; ++i) cc[i] = (int)(c0 + i < outc ? c0 + i : outc - 1);
#pragma unroll 4
  for (int s = 0; s < p.split_k; ++s) {
    const float* src = p.partials + ((int64_t)s * p.m + row) * ncols;
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
      v[i] += src[cc[i]];
      if (kSwiglu) u[i] += src[cc[i] + p.n];
    }
  }
  // per-token FP8 row scale (of the gathered token for gathered rows)
  const float rsc = row_act_scale<FMT>(p, row);
  if constexpr (EPI == EPI_BF16 || EPI == EPI_SCATTER) {
    uint16_t* out = static_cast<uint16_t*>(p.out);
    const int64_t orow = (EPI == EPI_SCATTER) ? (int64_t)p.sorted[row] : row;
    uint32_t h[kCols];
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
      float x = v[i] * col_scale<FMT>(wmeta, cc[i], gs) * rsc;
      if (EPI == EPI_BF16 && p.bias) x += bf16_bits_to_f32(p.bias[cc[i]]);
      h[i] = f32_to_bf16_bits(x);
    }
    uint16_t* dst = out + orow * p.ldo + c0;
    if (c0 + kCols <= outc && ((uintptr_t)dst & 15) == 0) {
      // a whole 16-byte group: one store
      u32x4_t w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = h[2 * i] | (h[2 * i + 1] << 16);
      *reinterpret_cast<u32x4_t*>(dst) = w;
    } else {
#pragma unroll
      for (int i = 0; i < kCols; ++i)
        if (c0 + i < outc) dst[i] = (uint16_t)h[i];
    }
  } else if constexpr (EPI == EPI_SWIGLU_BF16) {
    uint16_t* out = static_cast<uint16_t*>(p.out);
#pragma unroll
    for (int i = 0; i < kCols; ++i)
      if (c0 + i < outc) {
        const float a = swiglu_val<FMT>(p, wmeta, gs, rsc, c0 + i, v[i], u[i]);
        keep_swiglu_f32(p, row, c0 + i, a);
        out[row * p.ldo + c0 + i] = (uint16_t)f32_to_bf16_bits(a);
      }
  } else {
    float a[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      a[i] = swiglu_val<FMT>(p, wmeta, gs, rsc, c0 + i, v[i], u[i]);
      keep_swiglu_f32(p, row, c0 + i, a[i]);
      amax = __builtin_fmaxf(amax, __builtin_fabsf(a[i]));
    }
    const int e = mx_scale_code(amax);
    const float inv = mx_inv_scale(e);
    uint8_t* outq = static_cast<uint8_t*>(p.out) + row * p.ldo + c0;
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      const uint32_t q = f32x2_to_e4m3x2(a[i] * inv, a[i + 1] * inv);
      outq[i] = (uint8_t)(q & 0xFF);
      outq[i + 1] = (uint8_t)(q >> 8);
    }
    static_cast<uint8_t*>(p.out_scale)[row * (p.ldo / 32) + c0 / 32] = (uint8_t)e;
  }
}

// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// Instances.  The compiled template instances are listed in tables spread
// over several translation units (compiled in parallel); launch_gemm looks a
// key up in all of them.

typedef void (*gemm_fn)(const GemmParams);
typedef void (*reduce_fn)(const GemmParams, int);

struct Instance {
  KernelKey key;
  gemm_fn fn;
  int threads;
};

struct InstanceTable {
  const Instance* p;
  int n;
};

// One table per translation unit.
InstanceTable instances_dense_a();
InstanceTable instances_dense_b();
InstanceTable instances_dense_c();
InstanceTable instances_dense_d();
InstanceTable instances_dense_sk();
InstanceTable instances_moe_a();
InstanceTable instances_moe_b();
InstanceTable instances_moe_c();

#define HUM_TABLE(name, arr) \
  InstanceTable name() { return InstanceTable{arr, (int)(sizeof(arr) / sizeof(arr[0]))}; }

#define HUM_STREAM(F, WN, KW, PF, AM, EP) \
  {{F, KIND_STREAM, 1, WN, 1, KW, AM, EP, 0}, stream_kernel<F, WN, KW, PF, AM, EP>, 64 * stream_waves(F, KW, AM, EP)}
#define HUM_TILE_S(F, WM, WN, AM, EP, S) \
  {{F, KIND_TILE, WM, WN, 4, 1, AM, EP, S}, tile_kernel<F, WM, WN, AM, EP, S>, 256}
#define HUM_TILE(F, WM, WN, AM, EP) HUM_TILE_S(F, WM, WN, AM, EP, 2)
// Stream-K variants of dense tiles (MS: 16 or 32)
#define HUM_TILE_SK(F, WM, WN, S, MS)                                                              \
  {{F, (MS) == 32 ? KIND_TILE32 : KIND_TILE, WM, WN, 4, 1, A_DIRECT, EPI_BF16, S, 1},              \
   tile_kernel<F, WM, WN, A_DIRECT, EPI_BF16, S, MS, true>, 256}
#define HUM_TILE32_S(F, WM, WN, S) \
  {{F, KIND_TILE32, WM, WN, 4, 1, A_DIRECT, EPI_BF16, S}, tile_kernel<F, WM, WN, A_DIRECT, EPI_BF16, S, 32>, 256}
// 32x32-block tiles (bf16 activations: INT and MXFP4 weights; INT's 128 x
// 256 tile would spill its per-K-block accumulators)
#define HUM_DENSE_TILE32_SET(F)                            \
  HUM_TILE32_S(F, 2, 2, 2),                                \
  HUM_TILE32_S(F, 2, 4, 2),                                \
  HUM_TILE32_S(F, 4, 2, 2),                                \
  HUM_TILE32_S(F, 4, 4, 2),                                \
  HUM_TILE32_S(F, 8, 2, 2),                                \
  HUM_TILE32_S(F, 2, 2, 3),                                \
  HUM_TILE32_S(F, 2, 4, 3),                                \
  HUM_TILE32_S(F, 4, 2, 3),                                \
  HUM_TILE32_S(F, 4, 4, 3)

// Ring depth in 1-KB weight fragments per sub-tile (8-bit fragments are 2 KB:
// half as many).  A CU keeps about 64-128 KB of weights in flight.
#define HUM_PF(F, n) (((F) == F_FP8 || (F) == F_FP8_BLOCK || fmt_w8_bf16(F) || fmt_fp6(F)) ? ((n) > 1 ? (n) / 2 : 1) : (n))
#define HUM_DENSE_SET(F)                                   \
  HUM_STREAM(F, 1, 8, HUM_PF(F, 8), A_DIRECT, EPI_BF16),   \
  HUM_STREAM(F, 1, 15, HUM_PF(F, 8), A_DIRECT, EPI_BF16),  \
  HUM_STREAM(F, 2, 8, HUM_PF(F, 8), A_DIRECT, EPI_BF16),   \
  HUM_STREAM(F, 2, 15, HUM_PF(F, 4), A_DIRECT, EPI_BF16),  \
  HUM_STREAM(F, 4, 8, HUM_PF(F, 4), A_DIRECT, EPI_BF16),   \
  HUM_STREAM(F, 4, 15, HUM_PF(F, 2), A_DIRECT, EPI_BF16),  \
  HUM_STREAM(F, 1, 4, HUM_PF(F, 8), A_DIRECT, EPI_BF16),   \
  HUM_DENSE_TILE_SET(F)

// Tile instances only (formats without a decode-kernel path)
#define HUM_DENSE_TILE_SET(F)                              \
  HUM_TILE(F, 1, 4, A_DIRECT, EPI_BF16),                   \
  HUM_TILE(F, 2, 2, A_DIRECT, EPI_BF16),                   \
  HUM_TILE(F, 2, 4, A_DIRECT, EPI_BF16),                   \
  HUM_TILE(F, 4, 2, A_DIRECT, EPI_BF16),                   \
  HUM_TILE(F, 4, 4, A_DIRECT, EPI_BF16),                   \
  HUM_TILE(F, 8, 2, A_DIRECT, EPI_BF16),                   \
  HUM_TILE(F, 8, 4, A_DIRECT, EPI_BF16),                   \
  HUM_TILE_S(F, 2, 2, A_DIRECT, EPI_BF16, 3),              \
  HUM_TILE_S(F, 2, 4, A_DIRECT, EPI_BF16, 3),              \
  HUM_TILE_S(F, 4, 2, A_DIRECT, EPI_BF16, 3),              \
  HUM_TILE_S(F, 4, 4, A_DIRECT, EPI_BF16, 3),              \
  HUM_TILE_S(F, 8, 2, A_DIRECT, EPI_BF16, 3)

// MoE tile instances: gate_up (gathered rows, EPI_UP) and down (rows in
// sorted order, scattered to flat slots); gathered and sorted rows with the
// plain epilogue (per sorted row) serve the stage export.
#define HUM_MOE_TILE_SET(F, EPI_UP)                        \
  HUM_TILE(F, 1, 4, A_GATHER, EPI_UP),                     \
  HUM_TILE(F, 2, 4, A_GATHER, EPI_UP),                     \
  HUM_TILE(F, 4, 4, A_GATHER, EPI_UP),                     \
  HUM_TILE(F, 8, 4, A_GATHER, EPI_UP),                     \
  HUM_TILE(F, 1, 4, A_DIRECT, EPI_SCATTER),                \
  HUM_TILE(F, 2, 4, A_DIRECT, EPI_SCATTER),                \
  HUM_TILE(F, 4, 4, A_DIRECT, EPI_SCATTER),                \
  HUM_TILE(F, 8, 4, A_DIRECT, EPI_SCATTER),                \
  HUM_TILE(F, 1, 4, A_GATHER, EPI_BF16),                   \
  HUM_TILE(F, 2, 4, A_GATHER, EPI_BF16),                   \
  HUM_TILE(F, 4, 4, A_GATHER, EPI_BF16),                   \
  HUM_TILE(F, 8, 4, A_GATHER, EPI_BF16),                   \
  HUM_TILE(F, 1, 4, A_SORTED, EPI_BF16),                   \
  HUM_TILE(F, 2, 4, A_SORTED, EPI_BF16),                   \
  HUM_TILE(F, 4, 4, A_SORTED, EPI_BF16),                   \
  HUM_TILE(F, 8, 4, A_SORTED, EPI_BF16)

#define HUM_MOE_SET(F, EPI_UP)                             \
  HUM_STREAM(F, 4, 8, 4, A_GATHER, EPI_UP),                \
  HUM_STREAM(F, 4, 8, 4, A_DIRECT, EPI_SCATTER),           \
  HUM_STREAM(F, 4, 15, 2, A_GATHER, EPI_UP),               \
  HUM_STREAM(F, 4, 15, 2, A_DIRECT, EPI_SCATTER),          \
  HUM_STREAM(F, 4, 8, 4, A_GATHER, EPI_BF16),              \
  HUM_STREAM(F, 4, 15, 2, A_GATHER, EPI_BF16),             \
  HUM_STREAM(F, 4, 8, 4, A_SORTED, EPI_BF16),              \
  HUM_STREAM(F, 4, 15, 2, A_SORTED, EPI_BF16),             \
  HUM_MOE_TILE_SET(F, EPI_UP)

}  // namespace hum
