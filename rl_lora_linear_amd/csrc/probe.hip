// Measurement probes for the chip's own peaks: a register-only bf16 MFMA loop
// (the matrix cores' sustained rate with no operand traffic, at whatever clock
// the chip holds under that load) and a streaming copy (HBM bandwidth).  The
// rooflines of the hot-path kernels are reported against these as well as
// against the published peaks.
#include "common.hpp"
#include "sgmv.hpp"

namespace lora {

constexpr int PROBE_WAVES = 8;    // two waves per SIMD
constexpr int PROBE_CHAINS = 4;   // independent accumulators per wave

__global__ __launch_bounds__(64 * PROBE_WAVES) void probe_mfma_kernel(int64_t iters,
                                                                       float* __restrict__ sink) {
  const int tid = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((tid + i) & 7));
    b[i] = (__bf16)(0.002f * (float)((tid * 3 + i) & 7));
  }
  f32x16 c[PROBE_CHAINS];
#pragma unroll
  for (int k = 0; k < PROBE_CHAINS; ++k)
#pragma unroll
    for (int g = 0; g < 16; ++g) c[k][g] = 0.f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < PROBE_CHAINS; ++k) c[k] = mfma32(a, b, c[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < PROBE_CHAINS; ++k)
#pragma unroll
    for (int g = 0; g < 16; ++g) s += c[k][g];
  if (tid == 0) sink[blockIdx.x] = s;   // keeps the loop live
}

// One pass, no grid stride: each thread moves COPY_U 16-byte vectors of one
// 256-thread x COPY_U block of the buffer, all loads issued before the stores.
constexpr int COPY_U = 8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * 256 * COPY_U + threadIdx.x;
  u32x4 v[COPY_U];
#pragma unroll
  for (int u = 0; u < COPY_U; ++u) {
    const int64_t i = base + u * 256;
    if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < COPY_U; ++u) {
    const int64_t i = base + u * 256;
    if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
  }
}

// Read-only stream: each thread XORs COPY_U 16-byte vectors (all loads in
// flight together) and the block writes one word, so the traffic is reads.
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src,
                                                         int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * 256 * COPY_U + threadIdx.x;
  u32x4 v[COPY_U];
#pragma unroll
  for (int u = 0; u < COPY_U; ++u) {
    const int64_t i = base + u * 256;
    v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0, 0, 0, 0};
  }
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < COPY_U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  x = __reduce_or_sync(0xffffffffffffffffull, x);
  if ((threadIdx.x & 63) == 0 && x == 0x9E3779B9u) sink[0] = x;   // keeps the loads live
}

}  // namespace lora

using namespace lora;
using namespace lora_host;

extern "C" {

int64_t lora_probe_mfma_flops_per_iter(int32_t blocks) {
  return (int64_t)blocks * PROBE_WAVES * PROBE_CHAINS * (2 * 32 * 32 * 16);
}

lora_status lora_probe_mfma(int64_t iters, int32_t blocks, float* sink, void* stream) {
  LORA_ARG_CHECK(iters >= 1 && blocks >= 1 && blocks <= (1 << 20) && sink != nullptr,
                 "probe_mfma: iters >= 1, 1 <= blocks <= 2^20 and a sink of blocks floats");
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(64 * PROBE_WAVES), 0,
                     (hipStream_t)stream, iters, sink);
  return launch_check("probe_mfma");
}

lora_status lora_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  LORA_ARG_CHECK(src && dst && bytes >= 0 && bytes % 16 == 0, "probe_copy: bytes a multiple of 16");
  LORA_ARG_CHECK(((uintptr_t)src | (uintptr_t)dst) % 16 == 0, "probe_copy: 16-byte aligned buffers");
  if (bytes == 0) return LORA_OK;
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)cdiv(n16, 256 * COPY_U)), dim3(256), 0,
                     (hipStream_t)stream, (const u32x4*)src, (u32x4*)dst, n16);
  return launch_check("probe_copy");
}

lora_status lora_probe_read(const void* src, int64_t bytes, void* sink, void* stream) {
  LORA_ARG_CHECK(src && sink && bytes >= 0 && bytes % 16 == 0 && (uintptr_t)src % 16 == 0,
                 "probe_read: 16-byte aligned src, bytes a multiple of 16, a sink");
  if (bytes == 0) return LORA_OK;
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)cdiv(n16, 256 * COPY_U)), dim3(256), 0,
                     (hipStream_t)stream, (const u32x4*)src, n16, (uint32_t*)sink);
  return launch_check("probe_read");
}

}  // extern "C"
