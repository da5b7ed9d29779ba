// Routed-expert glue for gfx950 (TPU RL note, section 12 "Mixture-of-experts,
// and where adapters attach": an adapter covering the MLP covers every
// expert's projections; tinker-ticks "Step time": every expert weight is
// touched).  The expert projections themselves run on the grouped GEMM and
// the segmented LoRA kernels over assignments sorted by (expert, adapter).
//
//   moe_route      top-k experts per token by raw fp32 logit (ties to the lower
//                  expert index), listed best first, with the softmax renormalised
//                  over the chosen k: w_k = exp(z_k - z_1) / sum_k' exp(z_k' - z_1).
//   moe_keys       composite key of assignment j = t*K + k: e*(n_ad + 1) + a, with
//                  a = n_ad ("no adapter") for adapter ids out of range.
//   moe_desc       per-key descriptor tables with a rank-0 entry for "no adapter".
//   moe_gather_w   routing weight of each sorted position.
//   moe_combine    out[t] = sum_k w[t,k] (a + b)[position of t*K + k] in fp32, in
//                  k order (deterministic), rounded once to bf16.
//   planes_scale   bf16 hi/lo planes of w[p] * (hi + lo).
#include "common.hpp"
#include "sgmv.hpp"

namespace lora {

// One wave per token; each lane holds the logits e = q*64 + lane.
template <int VPL>
__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits,
                                                        int64_t n, int E, int K,
                                                        int32_t* __restrict__ experts,
                                                        float* __restrict__ weights) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= n) return;
  const float* row = logits + t * E;
  float v[VPL];
  uint32_t taken = 0;
#pragma unroll
  for (int q = 0; q < VPL; ++q) {
    const int e = q * 64 + lane;
    v[q] = e < E ? row[e] : -INFINITY;
    if (e >= E) taken |= 1u << q;
  }
  float my_v = -INFINITY, top = 0.f;
  int my_i = -1;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      const int e = q * 64 + lane;
      if (!((taken >> q) & 1u) && (v[q] > bv || (v[q] == bv && e < bi))) {
        bv = v[q];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (k == 0) top = bv;
    if (lane == k) {
      my_v = bv;
      my_i = bi;
    }
  }
  const float ex = lane < K ? expf(my_v - top) : 0.f;
  float sum = ex;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane < K) {
    experts[t * K + lane] = my_i;
    weights[t * K + lane] = ex / sum;
  }
}

__global__ __launch_bounds__(256) void moe_keys_kernel(const int32_t* __restrict__ experts,
                                                       const int32_t* __restrict__ ids,
                                                       int64_t n_assign, int K, int E, int n_ad,
                                                       int32_t* __restrict__ keys,
                                                       int32_t* status) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= n_assign) return;
  const int e = experts ? experts[j] : 0;   // null: one expert
  int a = ids[j / K];
  int key = -1;   // expert out of range: dropped (the segment builder flags it)
  if (e >= 0 && e < E) {
    if (a < 0 || a >= n_ad) {
      set_flag(status, LORA_FLAG_ID_RANGE);
      a = n_ad;
    }
    key = e * (n_ad + 1) + a;
  }
  keys[j] = key;
}

// blockIdx.y = table (gate, up, down)
struct DescTabs {
  const lora_adapter_desc* src[3];
  lora_adapter_desc* dst[3];
};
__global__ __launch_bounds__(256) void moe_desc_kernel(DescTabs tabs, int E, int n_ad) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  const int n_keys = E * (n_ad + 1);
  if (k >= n_keys) return;
  const int e = k / (n_ad + 1), a = k - e * (n_ad + 1);
  lora_adapter_desc d{0, 0, 0, 0.f};
  if (a < n_ad) d = tabs.src[blockIdx.y][e * n_ad + a];
  tabs.dst[blockIdx.y][k] = d;
}

__global__ __launch_bounds__(256) void moe_gather_w_kernel(const float* __restrict__ w,
                                                           const int32_t* __restrict__ perm,
                                                           int64_t n, float* __restrict__ wpos) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p < n) wpos[p] = w[perm[p]];
}

// One block per token; 8 columns (16 bytes of bf16) per thread and step.
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t* __restrict__ a,
                                                          const float* __restrict__ w,
                                                          const int32_t* __restrict__ inv,
                                                          const int32_t* __restrict__ keys,
                                                          int K, int64_t H,
                                                          uint16_t* __restrict__ out) {
  const int64_t t = blockIdx.x;
  for (int64_t c = (int64_t)threadIdx.x * 8; c < H; c += 256 * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
      const int64_t j = t * K + k;
      if (keys[j] < 0) continue;   // dropped assignments (invalid expert) add nothing
      const int64_t p = inv[j];
      const float wk = w ? w[j] : 1.f;
      const uint4 va = *(const uint4*)(a + p * H + c);
      const uint32_t xa[4] = {va.x, va.y, va.z, va.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += wk * bf2f_lo(xa[q]);
        acc[2 * q + 1] += wk * bf2f_hi(xa[q]);
      }
    }
    *(uint4*)(out + t * H + c) = make_uint4(pack2bf(acc[0], acc[1]), pack2bf(acc[2], acc[3]),
                                            pack2bf(acc[4], acc[5]), pack2bf(acc[6], acc[7]));
  }
}

// dst planes = split(w[p] * (hi + lo)); R (row length) a multiple of 2.
__global__ __launch_bounds__(256) void planes_scale_kernel(const uint16_t* __restrict__ src,
                                                           const float* __restrict__ wpos,
                                                           int64_t n, int R, int64_t plane,
                                                           uint16_t* __restrict__ dst) {
  const int64_t e2 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 2;
  if (e2 >= n * R) return;
  const int64_t p = e2 / R;
  const uint32_t hi = *(const uint32_t*)(src + e2), lo = *(const uint32_t*)(src + plane + e2);
  const float w = wpos[p];
  uint32_t h2, l2;
  split2_bf16(w * (bf2f_lo(hi) + bf2f_lo(lo)), w * (bf2f_hi(hi) + bf2f_hi(lo)), h2, l2);
  *(uint32_t*)(dst + e2) = h2;
  *(uint32_t*)(dst + plane + e2) = l2;
}

}  // namespace lora

namespace lora_host {
using namespace lora;

lora_status launch_moe_route(const float* logits, int64_t n, int E, int K, int32_t* experts,
                             float* weights, hipStream_t s) {
  if (n <= 0) return LORA_OK;
  const dim3 grid((unsigned)cdiv(n, 4));
  if (E <= 64)
    hipLaunchKernelGGL(moe_route_kernel<1>, grid, dim3(256), 0, s, logits, n, E, K, experts, weights);
  else if (E <= 128)
    hipLaunchKernelGGL(moe_route_kernel<2>, grid, dim3(256), 0, s, logits, n, E, K, experts, weights);
  else if (E <= 256)
    hipLaunchKernelGGL(moe_route_kernel<4>, grid, dim3(256), 0, s, logits, n, E, K, experts, weights);
  else
    hipLaunchKernelGGL(moe_route_kernel<16>, grid, dim3(256), 0, s, logits, n, E, K, experts, weights);
  return launch_check("moe_route");
}

lora_status launch_moe_keys(const int32_t* experts, const int32_t* ids, int64_t n_assign, int K,
                            int E, int n_ad, int32_t* keys, int32_t* status, hipStream_t s) {
  if (n_assign <= 0) return LORA_OK;
  hipLaunchKernelGGL(moe_keys_kernel, dim3((unsigned)cdiv(n_assign, 256)), dim3(256), 0, s, experts,
                     ids, n_assign, K, E, n_ad, keys, status);
  return launch_check("moe_keys");
}

lora_status launch_moe_desc(const lora_adapter_desc* const src[3], lora_adapter_desc* const dst[3],
                            int E, int n_ad, hipStream_t s) {
  DescTabs t{};
  for (int i = 0; i < 3; ++i) {
    t.src[i] = src[i];
    t.dst[i] = dst[i];
  }
  hipLaunchKernelGGL(moe_desc_kernel, dim3((unsigned)cdiv((int64_t)E * (n_ad + 1), 256), 3),
                     dim3(256), 0, s, t, E, n_ad);
  return launch_check("moe_desc");
}

lora_status launch_moe_gather_w(const float* w, const int32_t* perm, int64_t n, float* wpos,
                                hipStream_t s) {
  if (n <= 0) return LORA_OK;
  hipLaunchKernelGGL(moe_gather_w_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, w, perm,
                     n, wpos);
  return launch_check("moe_gather_w");
}

lora_status launch_moe_combine(const uint16_t* a, const float* w, const int32_t* inv,
                               const int32_t* keys, int64_t n_tok, int K, int64_t H,
                               uint16_t* out, hipStream_t s) {
  if (n_tok <= 0) return LORA_OK;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)n_tok), dim3(256), 0, s, a, w, inv, keys,
                     K, H, out);
  return launch_check("moe_combine");
}

lora_status launch_planes_scale(const uint16_t* src, const float* wpos, int64_t n, int R,
                                uint16_t* dst, hipStream_t s) {
  if (n <= 0) return LORA_OK;
  hipLaunchKernelGGL(planes_scale_kernel, dim3((unsigned)cdiv(n * R / 2, 256)), dim3(256), 0, s,
                     src, wpos, n, R, n * R, dst);
  return launch_check("planes_scale");
}

}  // namespace lora_host
