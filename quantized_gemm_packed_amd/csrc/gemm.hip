// Quantized GEMM launch: kernel instance lookup, split-K reduce instances,
// and the INT row-sum pre-pass.  The kernels (stream_kernel, tile_kernel,
// splitk_reduce_kernel) are templates in gemm_kernels.h; their compiled
// instances are listed in the inst_*.hip translation units.
#include "gemm_kernels.h"

#include <mutex>
#include <vector>

namespace hum {

// ---------------------------------------------------------------------------
// Row sums of bf16 activations per K-block (the INT prefill offset term), as
// bf16 hi / lo pairs in the A-operand layout the tile kernel reads (rows
// padded to 16, K-blocks to 32, with zeros).

__global__ __launch_bounds__(256) void rowsum_kernel(const uint16_t* __restrict__ a, int64_t lda, int64_t m,
                                                     int kb_count, int kbc, int64_t mt16,
                                                     uint16_t* __restrict__ out) {
  // one DPP row of 16 lanes per (row, K-block), K-blocks fastest: each lane
  // sums 8 values
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t item = gid >> 4;
  const int c = (int)(gid & 15);
  const int64_t kbp = (int64_t)kbc * 32;
  const bool in = item < mt16 * 16 * kbp;
  const int64_t row = in ? item / kbp : 0, kb = in ? item % kbp : 0;
  float s = 0.0f;
  if (in && row < m && kb < kb_count) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a + row * lda + kb * 128 + c * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) s += bf16_bits_to_f32(v[q] & 0xFFFF) + bf16_bits_to_f32(v[q] >> 16);
  }
  s = row16_sum(s);
  if (in && c == 0) {
    const uint32_t hi = f32_to_bf16_bits(s);
    const uint32_t lo = f32_to_bf16_bits(s - bf16_bits_to_f32(hi));
    const int64_t idx = (((row >> 4) * kbc + (kb >> 5)) * 64 + (row & 15) + 16 * ((kb >> 3) & 3)) * 8 + (kb & 7);
    out[idx] = (uint16_t)hi;
    out[mt16 * kbc * 512 + idx] = (uint16_t)lo;
  }
}

hum_status launch_rowsum(const void* a, int64_t lda, int64_t m, int kb_count, int kbc, uint8_t* out, void* stream) {
  if (m == 0) return HUM_OK;
  const int64_t mt16 = (m + 15) / 16;
  const int64_t threads = mt16 * 16 * (int64_t)kbc * 32 * 16;
  rowsum_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint16_t*>(a), lda, m, kb_count, kbc, mt16, reinterpret_cast<uint16_t*>(out));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "rowsum launch: %s", hipGetErrorString(err));
  return HUM_OK;
}

// ---------------------------------------------------------------------------
// Split-K reduce instances and the launcher.

struct ReduceInstance {
  int fmt, epi;
  reduce_fn fn;
};

static const ReduceInstance kReduces[] = {
    {F_INT, EPI_BF16, splitk_reduce_kernel<F_INT, EPI_BF16>},
    {F_INT3, EPI_BF16, splitk_reduce_kernel<F_INT3, EPI_BF16>},
    {F_INT2, EPI_BF16, splitk_reduce_kernel<F_INT2, EPI_BF16>},
    {F_INT1, EPI_BF16, splitk_reduce_kernel<F_INT1, EPI_BF16>},
    {F_MXFP6_BF16, EPI_BF16, splitk_reduce_kernel<F_MXFP6_BF16, EPI_BF16>},
    {F_MXBF6_BF16, EPI_BF16, splitk_reduce_kernel<F_MXBF6_BF16, EPI_BF16>},
    {F_FP8, EPI_BF16, splitk_reduce_kernel<F_FP8, EPI_BF16>},
    {F_MXFP4_BF16, EPI_BF16, splitk_reduce_kernel<F_MXFP4_BF16, EPI_BF16>},
    {F_MXFP4_BF16, EPI_SWIGLU_BF16, splitk_reduce_kernel<F_MXFP4_BF16, EPI_SWIGLU_BF16>},
    {F_MXFP4_BF16, EPI_SCATTER, splitk_reduce_kernel<F_MXFP4_BF16, EPI_SCATTER>},
    {F_MXFP4_MXFP8, EPI_BF16, splitk_reduce_kernel<F_MXFP4_MXFP8, EPI_BF16>},
    {F_MXFP4_MXFP4, EPI_BF16, splitk_reduce_kernel<F_MXFP4_MXFP4, EPI_BF16>},
    {F_FP8_BLOCK, EPI_BF16, splitk_reduce_kernel<F_FP8_BLOCK, EPI_BF16>},
    {F_FP8_BF16, EPI_BF16, splitk_reduce_kernel<F_FP8_BF16, EPI_BF16>},
    {F_INT8_BF16, EPI_BF16, splitk_reduce_kernel<F_INT8_BF16, EPI_BF16>},
    {F_NVFP4_BF16, EPI_BF16, splitk_reduce_kernel<F_NVFP4_BF16, EPI_BF16>},
    {F_MXINT4_BF16, EPI_BF16, splitk_reduce_kernel<F_MXINT4_BF16, EPI_BF16>},
    {F_MXFP4_MXFP8, EPI_SWIGLU_MXFP8, splitk_reduce_kernel<F_MXFP4_MXFP8, EPI_SWIGLU_MXFP8>},
    {F_MXFP4_MXFP8, EPI_SCATTER, splitk_reduce_kernel<F_MXFP4_MXFP8, EPI_SCATTER>},
#define HUM_MOE_REDUCES(F) {F, EPI_SWIGLU_BF16, splitk_reduce_kernel<F, EPI_SWIGLU_BF16>}, \
                           {F, EPI_SCATTER, splitk_reduce_kernel<F, EPI_SCATTER>}
    HUM_MOE_REDUCES(F_FP8),
    HUM_MOE_REDUCES(F_FP8_BLOCK),
    HUM_MOE_REDUCES(F_FP8_BF16),
    HUM_MOE_REDUCES(F_INT8_BF16),
    HUM_MOE_REDUCES(F_NVFP4_BF16),
    HUM_MOE_REDUCES(F_MXINT4_BF16),
#undef HUM_MOE_REDUCES
};

static const Instance* find_instance(const KernelKey& k) {
  static const InstanceTable tables[] = {instances_dense_a(), instances_dense_b(), instances_dense_c(),
                                         instances_dense_d(), instances_dense_sk(), instances_moe_a(),
                                         instances_moe_b(), instances_moe_c()};
  for (const InstanceTable& t : tables)
    for (int i = 0; i < t.n; ++i) {
      const KernelKey& q = t.p[i].key;
      if (q.fmt == k.fmt && q.kind == k.kind && q.wm == k.wm && q.wn == k.wn && q.waves_n == k.waves_n &&
          q.waves_k == k.waves_k && q.amode == k.amode && q.epi == k.epi && q.stages == k.stages && q.sk == k.sk)
        return &t.p[i];
    }
  return nullptr;
}

// Stream kernels whose dynamic-LDS limit was raised (once per kernel).
static std::mutex g_lds_mu;
static std::vector<const void*> g_big_lds;

bool gemm_instance_exists(const KernelKey& key) { return find_instance(key) != nullptr; }

bool reduce_instance_exists(int fmt, int epi) {
  for (const ReduceInstance& q : kReduces)
    if (q.fmt == fmt && q.epi == epi) return true;
  return false;
}

hum_status launch_gemm(const KernelKey& key, const GemmParams& p_in, int64_t m_tiles, int block_m, void* stream) {
  GemmParams p = p_in;
  if (p.group_m < 1) p.group_m = 1;
  p.a_gather = key.amode == A_GATHER;
  const Instance* in = find_instance(key);
  if (!in)
    return set_error(HUM_ERR_UNSUPPORTED,
                     "no GEMM instance fmt=%d kind=%d wm=%d wn=%d waves_n=%d waves_k=%d amode=%d epi=%d stages=%d",
                     key.fmt, key.kind, key.wm, key.wn, key.waves_n, key.waves_k, key.amode, key.epi, key.stages);
  const int64_t grid = p.sk_groups > 0 ? (int64_t)p.sk_groups : m_tiles * (int64_t)p.n_tiles * p.split_k;
  if (p.sk_groups > 0 && (key.kind == KIND_STREAM || p.split_k != 1 || key.amode != A_DIRECT || key.epi != EPI_BF16))
    return set_error(HUM_ERR_UNSUPPORTED, "Stream-K runs the dense tile kernels without split-K");
  if (grid <= 0) return HUM_OK;
  if (grid > 0x7FFFFFFF) return set_error(HUM_ERR_UNSUPPORTED, "grid too large");
  // buffer resources take 32-bit sizes and offsets
  constexpr int64_t kRsrcMax = (int64_t)1 << 31;
  if (p.a_bytes >= kRsrcMax || p.a_scale_bytes >= kRsrcMax)
    return set_error(HUM_ERR_UNSUPPORTED, "activations above 2 GiB");
  if (p.scales_per_expert >= kRsrcMax ||
      (p.wzero && (int64_t)(p.wzero - p.wscale) + p.zeros_per_expert >= kRsrcMax))
    return set_error(HUM_ERR_UNSUPPORTED, "weight metadata above 2 GiB");
  // the split-K reduce is resolved before anything is enqueued, so that a
  // configuration without one is refused with nothing launched
  const ReduceInstance* red_in = nullptr;
  if (p.split_k > 1) {
    for (const ReduceInstance& q : kReduces)
      if (q.fmt == key.fmt && q.epi == key.epi) red_in = &q;
    if (!red_in) return set_error(HUM_ERR_UNSUPPORTED, "no split-K reduce for fmt=%d epi=%d", key.fmt, key.epi);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  size_t dyn = 0;
  if (key.kind == KIND_STREAM) {
    const StreamLdsPlan L = stream_lds_plan(key.fmt, p.stream_rows, p.kb_per_split, key.wn, p.kb_per_group,
                                            p.scale_f32, p.ng, p.kb4);
    if (stream_self_staged(key.fmt, key.amode, key.epi) &&
        !stream_self_stage_fits(key.fmt, p.stream_rows, p.kb_per_split, key.waves_k, p.kb_per_group, p.scale_f32))
      return set_error(HUM_ERR_UNSUPPORTED, "stream kernel: K range per wave too long (raise split_k)");
    // (block-scaled FP8 rows are quantized in the kernel, four code chunks per lane)
    if (key.fmt == F_FP8_BLOCK && !stream_fp8_fuse_fits(p.stream_rows, p.kb_per_split, key.waves_k))
      return set_error(HUM_ERR_UNSUPPORTED, "stream kernel: K range per wave too long (raise split_k)");
    p.lds_meta_off = (int)L.meta_off;
    p.lds_meta_stride = (int)L.meta_stride;
    p.lds_zero_off = (int)L.zero_off;
    const int64_t red = (int64_t)(key.waves_k - 1) * key.wn * 64 * 16;
    dyn = (size_t)(L.total > red ? L.total : red);
    if ((int64_t)dyn > kStreamLdsMax) return set_error(HUM_ERR_UNSUPPORTED, "stream kernel: K range per split too long for LDS");
    if (dyn > 64 * 1024) {
      const void* fn = reinterpret_cast<const void*>(in->fn);
      std::lock_guard<std::mutex> lock(g_lds_mu);
      bool raised = false;
      for (const void* q : g_big_lds) raised = raised || q == fn;
      if (!raised) {
        if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStreamLdsMax) != hipSuccess)
          return set_error(HUM_ERR_HIP, "cannot raise the LDS limit of the stream kernel");
        g_big_lds.push_back(fn);
      }
    }
  }
  dim3 g((unsigned)grid);
  if (key.kind == KIND_STREAM) {
    if (m_tiles > 65535) return set_error(HUM_ERR_UNSUPPORTED, "stream kernel: more than 65535 row tiles");
    g = dim3((unsigned)p.n_tiles, (unsigned)m_tiles, (unsigned)p.split_k);
  }
  hipLaunchKernelGGL(in->fn, g, dim3(in->threads), dyn, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(HUM_ERR_HIP, "gemm launch: %s", hipGetErrorString(err));
  if (p.split_k > 1) {
    const ReduceInstance* r = red_in;
    const int64_t cols = (key.epi == EPI_SWIGLU_MXFP8) ? 32 : 8;
    const int64_t threads = p.m * ((p.n + cols - 1) / cols);
    if (threads > 0) {
      hipLaunchKernelGGL(r->fn, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p, block_m);
      err = hipGetLastError();
      if (err != hipSuccess) return set_error(HUM_ERR_HIP, "split-K reduce launch: %s", hipGetErrorString(err));
    }
  }
  return HUM_OK;
}

}  // namespace hum
