// Internal launchers of the segmented LoRA kernels, the GEMM and the
// elementwise kernels (host side).
#pragma once
#include "common.hpp"

namespace lora_host {

lora_status gemm_nt_bf16(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                         int64_t lda, int64_t ldb, int64_t ldc, hipStream_t s, int group_m = 0);
// Row gather/scatter through perm and the fused LoRA expand of the base GEMM.
struct LoraFuse {
  const int32_t* perm;      // segment order -> token
  const uint16_t* vec;      // per-token scaled vector: bf16 hi plane [tokens][vec_ld],
  int64_t vec_plane;        // lo plane at vec + vec_plane
  int vec_ld;
  int use_b_off;            // factor at b_off (B_a [N][r]) or a_off (A_a^T [N][r])
  const uint16_t* lmat;
  const lora_adapter_desc* desc;
  const int32_t* adpos;     // [tokens] adapter of each segment position, -1 for none
  int n_ad;
};
lora_status gemm_nt_lora(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                         int64_t lda, int64_t ldb, int64_t ldc, const LoraFuse& f, hipStream_t s,
                         int group_m = 0);
lora_status gemm_nt_lse(const uint16_t* A, const uint16_t* B, int M, int N, int K, int64_t lda,
                        int64_t ldb, float* part_m, float* part_s, float* zt,
                        const int32_t* targets, hipStream_t s, int group_m = 0);
lora_status gemm_nt_grad(const uint16_t* A, const uint16_t* B, uint16_t* G, int64_t ldg, int M,
                         int N, int K, int64_t lda, int64_t ldb, const int32_t* targets,
                         const float* lse, const float* dlogp, hipStream_t s, int group_m = 0);

lora_status launch_shrink(const uint16_t* in, int64_t ld_in, int K, const uint16_t* mat_pack,
                          int use_b_off, const lora_adapter_desc* desc, const int32_t* adpos,
                          const int32_t* perm, const int32_t* offsets, const int32_t* pre32,
                          int n_ad, int64_t n_tokens, uint16_t* out, int r_max, void* zero,
                          hipStream_t s);
lora_status launch_grad(int mode, const uint16_t* P, int r_max, const void* zero,
                        const uint16_t* Q, int64_t ld_q, int D, const lora_adapter_desc* desc,
                        const uint8_t* active, const int32_t* perm, const int32_t* offsets,
                        const int32_t* chunk_pre, int n_ad, int64_t n_tokens, float* out_pack,
                        float* partial, int accumulate, hipStream_t s);
int64_t grad_partial_floats(int64_t n_tokens, int n_ad, int64_t D, int r_max);
lora_status launch_adapter_transpose(const uint16_t* A_pack, const uint16_t* B_pack,
                                     const lora_adapter_desc* desc, const uint8_t* active,
                                     int n_ad, int64_t d_in, int64_t d_out, uint16_t* AT,
                                     uint16_t* BT, hipStream_t s);

constexpr int kGradChunk = 1024;  // tokens per gradient chunk (matches the kernel)

// ops.hip
lora_status launch_logprob_merge(const float* part_m, const float* part_s, const float* zt,
                                 const int32_t* targets, int64_t n, int tiles, int64_t vocab,
                                 float* logprobs, float* lse, int32_t* status, hipStream_t s);
lora_status launch_loss(int kind, int64_t n, const float* logp, const float* w, const float* adv,
                        const float* samp, const float* g, float clip_lo, float clip_hi,
                        double* partial, float* loss_out, float* dlogp, hipStream_t s);
lora_status launch_adam(int64_t n, float* p, const float* g, float* m, float* v, float lr,
                        float beta1, float beta2, float eps, float wd, float step_size,
                        float inv_sqrt_bc2, uint16_t* p_bf16, hipStream_t s);
lora_status launch_adam_multi(int n_seg, const int64_t* off, const int64_t* cnt,
                              const float* step_size, const float* inv_sqrt_bc2, float* p,
                              const float* g, float* m, float* v, float lr, float beta1,
                              float beta2, float eps, float wd, uint16_t* p_bf16, hipStream_t s);
lora_status launch_swiglu_fwd(int64_t n, const uint16_t* g, const uint16_t* u, uint16_t* h,
                              hipStream_t s);
lora_status launch_swiglu_bwd(int64_t n, const uint16_t* dh, const uint16_t* g,
                              const uint16_t* u, uint16_t* dg, uint16_t* du, hipStream_t s);
lora_status launch_transpose_bf16(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t cols,
                                  hipStream_t s);
lora_status launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

}  // namespace lora_host
