// Internal launchers of the segmented LoRA kernels, the GEMM and the
// elementwise kernels (host side).
#pragma once
#include "common.hpp"

namespace lora_host {

lora_status gemm_nt_bf16(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                         int64_t lda, int64_t ldb, int64_t ldc, hipStream_t s, int group_m = 0);
// Row maps, row groups and the fused LoRA expand of the base GEMM.  Position m
// (0 <= m < M) reads A row a_rows[m] and writes C row c_rows[m] (identity when
// null); rowscale[m] scales its base product.  With g_tile set, positions form
// n_groups consecutive groups (experts), group g = [g_off[g*g_stride],
// g_off[(g+1)*g_stride]) with its own B at B + g*ldb_group, tiled from
// g_tile[g]; tiles_m_bound bounds g_tile[n_groups].  With vec set, the expand
// adds (s u) . M_a^T from the bf16 hi/lo planes (lo at vec + vec_plane, row
// c_rows[m]) and the factor M_a at (use_b_off ? b_off : a_off) of lmat, for
// a = adpos[m] (-1: none).
struct GemmRows {
  const int32_t* a_rows = nullptr;
  int64_t a_rows_bound = 0;   // rows of A (checks the 32-bit gather offsets)
  const int32_t* c_rows = nullptr;
  const float* rowscale = nullptr;
  const int32_t* g_tile = nullptr;
  const int32_t* g_off = nullptr;
  int g_stride = 1;
  int n_groups = 0;
  int64_t ldb_group = 0;
  int tiles_m_bound = 0;
  const uint16_t* vec = nullptr;
  int64_t vec_plane = 0;
  int vec_ld = 0;
  int vec_by_pos = 0;       // vec rows are positions (else the C rows)
  int use_b_off = 0;        // 1: M_a = B_a [N][r] at b_off; 0: A_a [r][lmat_ld] at a_off
  int64_t lmat_ld = 0;
  const uint16_t* lmat = nullptr;
  const lora_adapter_desc* desc = nullptr;
  // Second weight operand B2 (same ldb / group stride as B), for
  //   k_split: K = k_split + K2 with k >= k_split read from B2 (both LoRA sets), or
  //   glu = 1 (below).
  const uint16_t* B2 = nullptr;
  int64_t c_off2 = 0;
  int k_split = 0;
  const uint16_t* vec2 = nullptr;
  const uint16_t* lmat2 = nullptr;
  const lora_adapter_desc* desc2 = nullptr;
  // SwiGLU epilogue: glu = 1, one launch writes [gate | up] rows to C (up at
  // column c_off2; B2 and LoRA set 2 for up) and hout = silu(gate) * up;
  // glu = 2, the product is dh (C nullable) and the epilogue writes dgu rows
  // [dgate | dup] from gu rows [gate | up] (second halves at c_off2).
  int glu = 0;
  uint16_t* hout = nullptr;
  int64_t ld_h = 0;
  const uint16_t* gu = nullptr;
  int64_t ld_gu = 0;
  uint16_t* dgu = nullptr;
  int64_t ld_dgu = 0;
  const int32_t* adpos = nullptr;
  int n_ad = 0;
};
lora_status gemm_nt_rows(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                         int64_t lda, int64_t ldb, int64_t ldc, const GemmRows& f, hipStream_t s,
                         int group_m = 0);
lora_status gemm_nt_lse(const uint16_t* A, const uint16_t* B, int M, int N, int K, int64_t lda,
                        int64_t ldb, float* part_m, float* part_s, float* zt,
                        const int32_t* targets, hipStream_t s, int group_m = 0);
lora_status gemm_nt_grad(const uint16_t* A, const uint16_t* B, uint16_t* G, int64_t ldg, int M,
                         int N, int K, int64_t lda, int64_t ldb, const int32_t* targets,
                         const float* lse, const float* dlogp, hipStream_t s, int group_m = 0);

// out[out_rows[p]] = bf16 hi/lo planes of s_a * rowscale[p] * (M_a in[in_rows[p]])
// over positions p < n_tokens (row maps and rowscale nullable), with M_a = A_a
// ([r][K] at a_off) or, from_b, M_a = B_a^T (B_a [K][r] at b_off, read in
// place); rows of positions without an adapter are zeroed, and `zero` (256 B,
// nullable) too.  Dual (mat_pack2 non-null, A factors, r_max <= 32): the same
// input rows also give out2 from the second table desc2 / mat_pack2.
lora_status launch_shrink(const uint16_t* in, int64_t ld_in, int K, const uint16_t* mat_pack,
                          int from_b, const lora_adapter_desc* desc, const int32_t* adpos,
                          const int32_t* in_rows, const int32_t* out_rows, const float* rowscale,
                          const int32_t* offsets, const int32_t* pre32, int n_ad,
                          int64_t n_tokens, uint16_t* out, int r_max, void* zero, hipStream_t s,
                          const uint16_t* mat_pack2 = nullptr,
                          const lora_adapter_desc* desc2 = nullptr, uint16_t* out2 = nullptr,
                          const int32_t* pre128 = nullptr, float* part = nullptr,
                          size_t part_floats = 0);
// (pre128 nullable: the prefix of ceil(count / 128) per key; with it, large
// batches run in 128-row tiles.  part nullable: with part_floats >=
// shrink_part_floats(n_tokens, n_ad, K) floats there, small batches split K
// over blocks and fold the chunk sums in a second launch; the bits of the
// result are the same either way.)
int shrink_split_parts(int64_t n_tokens, int n_ad, int K);
size_t shrink_part_floats(int64_t n_tokens, int n_ad, int K);
// Per key a: T_a = sum over a's positions p of P[p_row] Q[q_rows[p]]^T (mode 0:
// [D][r] at b_off; mode 1: [r][D] at a_off), P the bf16 hi/lo planes.  P row:
// the position itself with p_ident, else q_rows[p].  q_rows nullable.
lora_status launch_grad(int mode, const uint16_t* P, int r_max, const void* zero,
                        const uint16_t* Q, int64_t ld_q, int D, const lora_adapter_desc* desc,
                        const uint8_t* active, const int32_t* q_rows, int p_ident,
                        const int32_t* offsets, const int32_t* chunk_pre, int n_ad,
                        int64_t n_tokens, float* out_pack, float* partial, int accumulate,
                        hipStream_t s, const uint16_t* P2 = nullptr,
                        const lora_adapter_desc* desc2 = nullptr, float* out2 = nullptr);
// Dual (mode 1, r_max <= 32): P2 (same layout as P, in the same allocation)
// with desc2 gives the second table's T into out2 in the same pass over Q;
// the partial buffer then needs grad_partial_floats(.., 2 * r_max).
int64_t grad_partial_floats(int64_t n_tokens, int n_ad, int64_t D, int r_max);
// dB (mode 0 over u and dy, [d_out][r] at b_off) and dA (mode 1 over v and x,
// [r][d_in] at a_off) of one layer in one launch, and one finalize launch;
// each side takes its own partial buffer of grad_partial_floats(.., its D, r_max).
lora_status launch_grad_pair(const uint16_t* u, const uint16_t* dy, int64_t ld_dy, int d_out,
                             float* dB_pack, float* partial_b, const uint16_t* v,
                             const uint16_t* x, int64_t ld_x, int d_in, float* dA_pack,
                             float* partial_a, int r_max, const void* zero,
                             const lora_adapter_desc* desc, const uint8_t* active,
                             const int32_t* q_rows, const int32_t* offsets,
                             const int32_t* chunk_pre, int n_ad, int64_t n_tokens, int accumulate,
                             hipStream_t s);


constexpr int kGradChunk = 1024;  // tokens per gradient chunk (matches the kernel)

// ops.hip
lora_status launch_logprob_merge(const float* part_m, const float* part_s, const float* zt,
                                 const int32_t* targets, int64_t n, int tiles, int64_t vocab,
                                 float* logprobs, float* lse, int32_t* status, hipStream_t s);
lora_status launch_loss(int kind, int64_t n, const float* logp, const float* w, const float* adv,
                        const float* samp, const float* g, float clip_lo, float clip_hi,
                        double* partial, float* loss_out, float* dlogp, int32_t* status,
                        hipStream_t s);
// skip: n_seg int32 per-segment flags (cleared, then 1 where the update is skipped)
lora_status launch_adam_multi(int n_seg, const int64_t* off, const int64_t* cnt,
                              const float* step_size, const float* inv_sqrt_bc2, float* p,
                              const float* g, float* m, float* v, float lr, float beta1,
                              float beta2, float eps, float wd, uint16_t* p_bf16, int32_t* skip,
                              int32_t* status, hipStream_t s);
lora_status launch_swiglu_fwd(int64_t n, const uint16_t* g, const uint16_t* u, uint16_t* h,
                              hipStream_t s);
lora_status launch_swiglu_bwd(int64_t n, const uint16_t* dh, const uint16_t* g,
                              const uint16_t* u, uint16_t* dg, uint16_t* du, hipStream_t s);
lora_status launch_add_bf16(int64_t n, const uint16_t* a, const uint16_t* b, uint16_t* out,
                            hipStream_t s);
lora_status launch_transpose_bf16(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t cols,
                                  hipStream_t s);
lora_status launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
// *dst |= *src (a status word into another), one tiny launch
lora_status launch_or_status(const int32_t* src, int32_t* dst, hipStream_t s);

// moe.hip
lora_status launch_moe_route(const float* logits, int64_t n, int E, int K, int32_t* experts,
                             float* weights, hipStream_t s);
lora_status launch_moe_keys(const int32_t* experts, const int32_t* ids, int64_t n_assign, int K,
                            int E, int n_ad, int32_t* keys, int32_t* status, hipStream_t s);
lora_status launch_moe_desc(const lora_adapter_desc* const src[3], lora_adapter_desc* const dst[3],
                            int E, int n_ad, hipStream_t s);
lora_status launch_moe_gather_w(const float* w, const int32_t* perm, int64_t n, float* wpos,
                                hipStream_t s);
lora_status launch_moe_combine(const uint16_t* a, const float* w, const int32_t* inv,
                               const int32_t* keys, int64_t n_tok, int K, int64_t H,
                               uint16_t* out, hipStream_t s);
lora_status launch_planes_scale(const uint16_t* src, const float* wpos, int64_t n, int R,
                                uint16_t* dst, hipStream_t s);

}  // namespace lora_host
