// Device peak probes for the measurement (not part of the GEMM path): the
// rooflines the bench reports are the published MI355X peaks, and these
// kernels re-measure what this machine sustains -- a stream read of a large
// buffer (HBM), and matrix-instruction issue loops for the bf16, FP8,
// FP4 and mixed E4M3 x E2M1 rates the GEMMs use.
#include "dev_common.h"
#include "hum_internal.h"

namespace hum {

// Every lane sums 16-byte words over a grid-stride walk of the buffer and
// writes one word, so that no load is dead.
__global__ __launch_bounds__(256) void peak_read_kernel(const u32x4_t* __restrict__ p, int64_t words,
                                                        uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < words; i += 4 * stride) {
    const u32x4_t a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < words; i += stride) {
    const u32x4_t a = p[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// KIND 0: bf16 16x16x32; 1: E4M3 x E4M3 16x16x128; 2: E2M1 x E2M1
// 16x16x128; 3: E4M3 x E2M1 16x16x128 (the W4A8 instruction); 4..7 the
// same with the 32x32 shapes (bf16 32x32x16, f8f6f4 32x32x64).  Eight
// (16x16) or four (32x32) independent accumulators per wave keep the
// matrix pipe busy.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
template <int KIND>
__global__ __launch_bounds__(256) void peak_mfma32_kernel(int64_t iters, float* __restrict__ sink) {
  f32x16_t c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[j][i] = 0.0f;
  const uint32_t seed = threadIdx.x * 0x9E3779B9u;
  i32x8_t b8;
#pragma unroll
  for (int j = 0; j < 8; ++j) b8[j] = (int)(seed ^ (0x01010101u * j)) & 0x3B3B3B3B;
  bf16x8_t a16 = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u ^ seed, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (KIND == 4)
        c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a16, a16, c[j], 0, 0, 0);
      else if constexpr (KIND == 5)
        c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, b8, c[j], 0, 0, 0, 127, 0, 127);
      else if constexpr (KIND == 6)
        c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, b8, c[j], 4, 4, 0, 127, 0, 127);
      else
        c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, b8, c[j], 0, 4, 0, 127, 0, 127);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += c[j][0] + c[j][15];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

template <int KIND>
__global__ __launch_bounds__(256) void peak_mfma_kernel(int64_t iters, float* __restrict__ sink) {
  f32x4_t c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const uint32_t seed = threadIdx.x * 0x9E3779B9u;
  i32x8_t b8;
#pragma unroll
  for (int j = 0; j < 8; ++j) b8[j] = (int)(seed ^ (0x01010101u * j)) & 0x3B3B3B3B;
  bf16x8_t a16 = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u ^ seed, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (KIND == 0)
        c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a16, a16, c[j], 0, 0, 0);
      else if constexpr (KIND == 1)
        c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, b8, c[j], 0, 0, 0, 127, 0, 127);
      else if constexpr (KIND == 2)
        c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, b8, c[j], 4, 4, 0, 127, 0, 127);
      else
        c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, b8, c[j], 0, 4, 0, 127, 0, 127);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace hum

using namespace hum;

extern "C" {

hum_status hum_peak_probe(int32_t kind, int64_t n, const void* buf, void* sink, double* work_out, void* stream) {
  clear_error();
  hipStream_t s = static_cast<hipStream_t>(stream);
  constexpr int kGrid = 256 * 8;  // eight workgroups of four waves per CU
  if (!sink || !work_out || n < 1) return set_error(HUM_ERR_INVALID_ARG, "bad probe arguments");
  if (kind == HUM_PEAK_HBM_READ) {
    if (!buf || n % 16) return set_error(HUM_ERR_INVALID_ARG, "read probe: buf and a multiple of 16 bytes");
    peak_read_kernel<<<kGrid, 256, 0, s>>>(static_cast<const u32x4_t*>(buf), n / 16, static_cast<uint32_t*>(sink));
    *work_out = (double)n;
  } else if (kind >= HUM_PEAK_MFMA32_BF16 && kind <= HUM_PEAK_MFMA32_FP8_FP4) {
    const int k = kind - HUM_PEAK_MFMA32_BF16;
    float* o = static_cast<float*>(sink);
    if (k == 0) peak_mfma32_kernel<4><<<kGrid, 256, 0, s>>>(n, o);
    if (k == 1) peak_mfma32_kernel<5><<<kGrid, 256, 0, s>>>(n, o);
    if (k == 2) peak_mfma32_kernel<6><<<kGrid, 256, 0, s>>>(n, o);
    if (k == 3) peak_mfma32_kernel<7><<<kGrid, 256, 0, s>>>(n, o);
    const double per_inst = k == 0 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
    *work_out = (double)kGrid * 4 * (double)n * 4 * per_inst;
  } else if (kind >= HUM_PEAK_MFMA_BF16 && kind <= HUM_PEAK_MFMA_FP8_FP4) {
    const int k = kind - HUM_PEAK_MFMA_BF16;
    float* o = static_cast<float*>(sink);
    if (k == 0) peak_mfma_kernel<0><<<kGrid, 256, 0, s>>>(n, o);
    if (k == 1) peak_mfma_kernel<1><<<kGrid, 256, 0, s>>>(n, o);
    if (k == 2) peak_mfma_kernel<2><<<kGrid, 256, 0, s>>>(n, o);
    if (k == 3) peak_mfma_kernel<3><<<kGrid, 256, 0, s>>>(n, o);
    const double per_inst = k == 0 ? 2.0 * 16 * 16 * 32 : 2.0 * 16 * 16 * 128;
    *work_out = (double)kGrid * 4 * (double)n * 8 * per_inst;
  } else {
    return set_error(HUM_ERR_INVALID_ARG, "unknown probe kind %d", kind);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "probe launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

}  // extern "C"
