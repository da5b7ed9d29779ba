/*
 * lora_mi355x.h -- C ABI of the mixed-adapter LoRA training hot path for
 * AMD MI355X (gfx950).
 *
 * What the library computes (sources are the pages' titles and sections):
 *   - Many users' LoRA adapters train in one batch over one frozen base weight
 *     (tinker-ticks, "Why multiplexing matters"; OpenTinker, abstract).  All
 *     tokens are flattened into one matrix with a per-row adapter id; the base
 *     product is one shared GEMM and the adapter delta is a segmented shrink
 *     (x A_i^T, down to rank r_i) followed by an expand (. B_i^T, back up)
 *     (tinker-ticks, "How the SGMV kernel works", "Forward pass: what actually
 *     happens").  The adapted weight is W + s_i B_i A_i with s_i = alpha_i/r_i
 *     (Deep Dive - Tinker, "LoRA is the adaptation boundary").
 *   - Backward produces dX and per-adapter dA_i, dB_i only; the base is frozen
 *     and each adapter's gradient sums only its own tokens (OpenTinker,
 *     "3 Approach"; TPU RL note, section 4).
 *   - Target-token logprobs through the lm_head with an online logsumexp that
 *     never writes the N x V logits, and a backward that recomputes logits
 *     chunk by chunk (TPU RL note, section 10, items 1, 3 and 4).
 *   - Token losses cross_entropy, importance_sampling, ppo and the custom
 *     dLoss/dlogprob path (Deep Dive - Tinker, "The RL datum shape";
 *     forward_backward_custom post).
 *   - Per-adapter AdamW with its own moments and step (Deep Dive - Tinker,
 *     "optim_step advances adapter state").
 *
 * Conventions
 *   - bf16 tensors are passed as uint16_t bit patterns; fp32 as float.
 *   - Every pointer is a DEVICE pointer unless its comment says host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work; they return before it runs.  Buffers must stay
 *     alive until the stream reaches the work.
 *   - Matrices are row-major.  W [d_out][d_in] (PyTorch Linear layout);
 *     adapter i has A_i [r_i][d_in] and B_i [d_out][r_i] at element offsets
 *     desc[i].a_off / desc[i].b_off of the A and B packs (the packs may be the
 *     same buffer).  Offsets are in elements and must be multiples of 8.
 *   - The caller owns every buffer, including the workspace `ws` sized by the
 *     matching *_workspace_bytes() call.  The library keeps no pointer after a
 *     call returns and allocates no device memory.  One workspace must not be
 *     used by two streams at once.  Word 0 of every workspace is a sticky
 *     status word: zero it once (lora_workspace_init or a zero-filled
 *     allocation); kernels OR device-detected content errors into it, and
 *     lora_device_status reads and clears it.
 *
 * Errors
 *   - Problems visible on the host (NULL pointers, bad sizes, unsupported
 *     shapes, a workspace that is too small) return a status before anything
 *     is enqueued; lora_last_error() then describes it (thread-local).
 *   - Content errors visible only on the device (ids or targets out of range,
 *     unsorted ids under LORA_IDS_SORTED, invalid adapter descriptors) set bits
 *     of the workspace status word.  Offending rows are never used as
 *     addresses: a token with an invalid adapter id gets the base output and
 *     contributes to no gradient; an invalid descriptor makes its adapter
 *     inactive (zero delta, zero gradient); an out-of-range target gives a NaN
 *     logprob and a zero dh row.
 *   - Non-finite values propagate per IEEE 754 through the projections and the
 *     logprob path.  Three places contain them (TPU RL note, section 12 "The
 *     instability I have not solved"): masked loss rows are removed by
 *     selection, never by multiplying by zero (inf * 0 is NaN); a kept loss
 *     row whose own inputs are non-finite is removed the same way and
 *     LORA_FLAG_NONFINITE_LOSS is set; an adapter whose gradient holds a
 *     non-finite element is not updated by AdamW at all and
 *     LORA_FLAG_NONFINITE_GRAD is set.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LORA_OK = 0,
  LORA_E_INVALID_ARG = 1,   /* NULL pointer, negative or inconsistent size */
  LORA_E_UNSUPPORTED = 2,   /* shape outside what the kernels handle (see each call) */
  LORA_E_WORKSPACE = 3,     /* workspace NULL or smaller than required */
  LORA_E_HIP = 4,           /* a HIP launch or runtime call failed */
  LORA_E_DEVICE_CHECK = 5   /* lora_device_status found content errors */
} lora_status;

/* Bits of the workspace status word. */
#define LORA_FLAG_ID_RANGE     0x1  /* an adapter/segment id outside [0, n_keys) */
#define LORA_FLAG_UNSORTED     0x2  /* ids decrease although LORA_IDS_SORTED was promised */
#define LORA_FLAG_TARGET_RANGE 0x4  /* a target token id outside [0, vocab) */
#define LORA_FLAG_BAD_DESC     0x8  /* an adapter descriptor with bad rank, offset or alignment */
#define LORA_FLAG_NONFINITE_GRAD 0x10 /* AdamW skipped an adapter whose gradient held NaN or Inf */
#define LORA_FLAG_NONFINITE_LOSS 0x20 /* loss_grad removed kept rows whose inputs held NaN or Inf */

typedef enum { LORA_IDS_SORTED = 0, LORA_IDS_INTERLEAVED = 1 } lora_id_order;

/* One adapter.  Device array of n_adapters entries (24 bytes each).
 * rank: 8..64 and a multiple of 8, and <= lora_shape.max_rank; 0 marks an unused
 * slot (the adapter is inactive, without a flag).
 * scale: s_i = alpha_i / r_i, applied to the LoRA delta and its gradients. */
typedef struct {
  int64_t a_off;   /* element offset of A_i [rank][d_in] in the A pack */
  int64_t b_off;   /* element offset of B_i [d_out][rank] in the B pack */
  int32_t rank;
  float scale;
} lora_adapter_desc;

/* Shape of one mixed-adapter layer call (host struct). */
typedef struct {
  int64_t n_tokens;      /* N >= 0 */
  int64_t d_in;          /* multiple of 64 */
  int64_t d_out;         /* multiple of 64 */
  int64_t a_pack_elems;  /* elements readable from the A pack (bound for descriptor checks) */
  int64_t b_pack_elems;  /* elements readable from the B pack */
  int32_t n_adapters;    /* 1 .. 16384 */
  int32_t max_rank;      /* 16 .. 64, multiple of 16: u/v row stride and rank bound */
  int32_t order;         /* lora_id_order: a promise about adapter_ids, checked on device */
  int32_t reserved;      /* must be 0 */
} lora_shape;

/* ---- workspace and status -------------------------------------------- */

/* Bytes of workspace lora_forward / lora_backward need for this shape. */
size_t lora_workspace_bytes(const lora_shape* shape);

/* Zero the status word of a workspace (enqueued on `stream`). */
lora_status lora_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Synchronise `stream`, copy the workspace status word to *host_flags (host
 * pointer) and clear it.  Returns LORA_E_DEVICE_CHECK if any bit was set. */
lora_status lora_device_status(void* ws, int32_t* host_flags, void* stream);

/* Description of the last host-side error on this thread ("" if none). */
const char* lora_last_error(void);

/* ---- segments --------------------------------------------------------- */

/* Stable counting sort of per-token keys (tinker-ticks, "How the SGMV kernel
 * works": one segment index per flattened row).
 *   ids     int32 [n]        keys; valid keys are 0..n_keys-1
 *   perm    int32 [n] out    tokens of key 0 in increasing index, then key 1,
 *                            ...; tokens with invalid keys last, in index order
 *   offsets int32 [n_keys+1] out  offsets[k]..offsets[k+1] is key k's range;
 *                            offsets[n_keys] = number of valid tokens
 * order = LORA_IDS_SORTED additionally flags LORA_FLAG_UNSORTED if ids
 * decrease anywhere.  Out-of-range ids set LORA_FLAG_ID_RANGE.
 * Requires n >= 0 (n = 0 writes offsets of zeros), 1 <= n_keys <= 16384 and a
 * workspace of lora_segments_workspace_bytes(n, n_keys). */
size_t lora_segments_workspace_bytes(int64_t n, int32_t n_keys);
lora_status lora_segments(const int32_t* ids, int64_t n, int32_t n_keys, int32_t order,
                          int32_t* perm, int32_t* offsets, void* ws, size_t ws_bytes,
                          void* stream);

/* ---- frozen-operand layout helper ----------------------------------- */

/* dst [cols][rows] = transpose of src [rows][cols] (bf16).  Frozen weights
 * are kept in both layouts so every GEMM reads K-contiguous operands: call it
 * once per frozen matrix (W for lora_backward, the lm_head for
 * token_logprobs_backward).  rows, cols multiples of 64; src != dst. */
lora_status lora_transpose_bf16(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t cols,
                                void* stream);

/* ---- mixed-adapter LoRA layer ---------------------------------------- */

/* Forward of the adapted layer over a mixed-adapter token batch:
 *   y_t = W x_t + s_a B_a (A_a x_t),   u_t = A_a x_t,   a = adapter_ids[t]
 * (tinker-ticks, "Forward pass: what actually happens", written in Linear
 * layout).
 *   x       bf16 [N][d_in]        W bf16 [d_out][d_in] (frozen)
 *   A_pack, B_pack bf16           desc lora_adapter_desc [n_adapters] (device)
 *   adapter_ids int32 [N]
 *   y       bf16 [N][d_out] out   (bf16 of the fp32-accumulated base product,
 *                                  then the fp32 delta added and rounded again)
 *   u_saved bf16 [2][N][max_rank] out  the scaled s_a u_t as two planes:
 *                                  plane 0 holds hi = bf16(s_a u_t), plane 1
 *                                  lo = bf16(s_a u_t - hi) (both round to
 *                                  nearest even), so hi + lo carries s_a u_t to
 *                                  ~2^-16 relative.  Columns r_a.. and rows of
 *                                  invalid tokens are zero.  4*N*max_rank
 *                                  bytes; keep it for lora_backward.
 * Tokens need not be sorted: LORA_IDS_INTERLEAVED gathers rows by adapter. */
lora_status lora_forward(const lora_shape* shape, const uint16_t* x, const uint16_t* W,
                         const uint16_t* A_pack, const uint16_t* B_pack,
                         const lora_adapter_desc* desc, const int32_t* adapter_ids,
                         uint16_t* y, uint16_t* u_saved, void* ws, size_t ws_bytes, void* stream);

/* Backward for upstream g = dL/dy (OpenTinker, "3 Approach": adapter-local
 * gradients; the base W is frozen so there is no dW):
 *   v_t   = B_a^T g_t
 *   dx_t  = W^T g_t + s_a A_a^T v_t
 *   dB_a  = s_a sum_{t in a} g_t u_t^T     dA_a = s_a sum_{t in a} v_t x_t^T
 *   dy      bf16 [N][d_out]      x bf16 [N][d_in]
 *   W_t     bf16 [d_in][d_out]   the frozen base weight TRANSPOSED (see
 *                                lora_transpose_bf16)
 *   u_saved bf16 [2][N][max_rank] from lora_forward with the same inputs
 *   dx      bf16 [N][d_in] out
 *   dA_pack, dB_pack fp32 out    same offsets as the A/B packs (may be one
 *                                buffer).  accumulate = 0 overwrites every
 *                                adapter's region (zeros for adapters with no
 *                                token); accumulate != 0 adds into it, which
 *                                is how gradients accumulate across calls
 *                                until the optimizer step (Deep Dive - Tinker,
 *                                "optim_step advances adapter state").
 * The per-adapter sums run in a fixed order: results are bitwise repeatable
 * and a token routed to adapter i never touches adapter j's gradient. */
lora_status lora_backward(const lora_shape* shape, const uint16_t* dy, const uint16_t* x,
                          const uint16_t* W_t, const uint16_t* A_pack, const uint16_t* B_pack,
                          const lora_adapter_desc* desc, const int32_t* adapter_ids,
                          const uint16_t* u_saved, uint16_t* dx, float* dA_pack, float* dB_pack,
                          int accumulate, void* ws, size_t ws_bytes, void* stream);

/* ---- fused lm_head + target logprob ----------------------------------- */

/* logprob_t = z_t[y_t] - lse_t with z_t = U h_t and lse_t = m + log sum exp(z - m)
 * (TPU RL note, section 10, "3 - Never materialize a log-softmax" and
 * "4 - Fused linear cross-entropy").  Logits are fp32 and never leave the
 * chip's registers/LDS; per (row, vocab tile) partial (max, sum) pairs are
 * merged in a fixed order.
 *   h bf16 [n][hidden]; lm_head bf16 [vocab][hidden]; targets int32 [n]
 *   logprobs, lse fp32 [n] out
 * hidden and vocab multiples of 64 below 2^30; 0 <= n < 2^30.  The size
 * queries return 0 for any n or vocab outside these ranges. */
size_t token_logprobs_workspace_bytes(int64_t n, int64_t vocab);
lora_status token_logprobs(int64_t n, int64_t hidden, int64_t vocab, const uint16_t* h,
                           const uint16_t* lm_head, const int32_t* targets, float* logprobs,
                           float* lse, void* ws, size_t ws_bytes, void* stream);

/* dh_t = dlogp_t (U[y_t] - sum_v softmax(z_t)_v U[v]), recomputing logits
 * token chunk by token chunk: G = dlogp (onehot - exp(z - lse)) is written as
 * bf16 for one chunk of rows at a time, then dh = G U (the custom-VJP shape
 * of the TPU RL note, section 10 item 4).  Rows with dlogp == 0 are exactly 0.
 *   lm_head_t bf16 [hidden][vocab]  the lm_head transposed (frozen)
 *   lse fp32 [n] from token_logprobs;  dlogp fp32 [n];  dh bf16 [n][hidden] out
 * The chunk is the largest multiple of 256 rows whose G fits the workspace;
 * token_logprobs_backward_workspace_bytes(n, vocab, rows) sizes one for a
 * chunk of `rows` (>= 256) rounded up to 256, capped at n rounded up to 256
 * (the longest chunk the call runs). */
size_t token_logprobs_backward_workspace_bytes(int64_t n, int64_t vocab, int64_t chunk_rows);
lora_status token_logprobs_backward(int64_t n, int64_t hidden, int64_t vocab, const uint16_t* h,
                                    const uint16_t* lm_head, const uint16_t* lm_head_t,
                                    const int32_t* targets, const float* lse, const float* dlogp,
                                    uint16_t* dh, void* ws, size_t ws_bytes, void* stream);

/* ---- token loss -------------------------------------------------------- */

typedef enum {
  LOSS_CROSS_ENTROPY = 0,        /* L = -sum w l;          dl = -w          */
  LOSS_IMPORTANCE_SAMPLING = 1,  /* rho = exp(l - l_s);  L = -sum rho A;  dl = -rho A */
  LOSS_PPO = 2,                  /* L = -sum min(rho A, clip(rho, 1-lo, 1+hi) A);
                                    dl = -rho A, or 0 where the clipped term is taken
                                    outside the (inclusive) clip range */
  LOSS_CUSTOM = 3                /* dl = g (external dLoss/dlogprob); reports S = sum g l */
} loss_kind;

typedef struct { float clip_low, clip_high; } loss_config;

/* Per-token loss gradient and the summed loss (Deep Dive - Tinker, "The RL
 * datum shape"; forward_backward_custom post; TPU RL note, section 12).
 *   logprobs fp32 [n]  current l
 *   weights  fp32 [n]  CROSS_ENTROPY: per-token weight w; other kinds: mask
 *                      (row kept iff != 0).  Rows with 0 get dl = 0 and no loss
 *                      term, by selection, whatever the other inputs hold.
 *   advantages, sampler_logprobs fp32 [n]  (IS, PPO; else may be NULL)
 *   custom_g fp32 [n]  (CUSTOM; else may be NULL)
 *   cfg      host pointer (PPO; else may be NULL)
 *   loss_out fp32 [1] out (device): deterministic sum, fixed order in fp64
 *   dlogp    fp32 [n] out
 * Sentinel (TPU RL note, section 12 "The instability I have not solved": a
 * NaN logprob is caught and its token gets a zero weight and a neutralised
 * value): a kept row any of whose inputs to its own term is NaN or +-Inf --
 * logprobs and weights for every kind, advantages and sampler_logprobs for
 * IS and PPO, custom_g for CUSTOM -- is removed by selection exactly like a
 * masked row (dlogp = 0, no loss term), and LORA_FLAG_NONFINITE_LOSS is set
 * in the workspace status word (read it with lora_device_status).  Inputs a
 * kind does not read are never inspected.  A finite row whose ratio
 * exp(l - l_s) overflows fp32 still follows IEEE 754.
 * 0 <= n < 2^30 (the size query returns 0 outside it).
 * Workspace: loss_grad_workspace_bytes(n); word 0 is the status word. */
size_t loss_grad_workspace_bytes(int64_t n);
lora_status loss_grad(int32_t kind, int64_t n, const float* logprobs, const float* weights,
                      const float* advantages, const float* sampler_logprobs,
                      const float* custom_g, const loss_config* cfg, float* loss_out,
                      float* dlogp, void* ws, size_t ws_bytes, void* stream);

/* ---- optimizer -------------------------------------------------------- */

/* One AdamW step on ONE adapter's flat fp32 parameters (Deep Dive - Tinker,
 * "optim_step advances adapter state": AdamW-equivalent, weight decay 0 by
 * default, moments kept per training client):
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;  p -= lr wd p;
 *   p -= (lr / (1 - b1^step)) m / (sqrt(v) / sqrt(1 - b2^step) + eps)
 * step >= 1 is this adapter's own counter (bias factors are computed on the
 * host in double).  p, m, v updated in place; g read only.  p_bf16 (nullable)
 * receives bf16(p) -- the bf16 copy the layer kernels read.  n >= 0.
 * Non-finite gradients (TPU RL note, section 12 "The instability I have not
 * solved": a non-finite optimizer update is skipped outright): if ANY element
 * of g is NaN or +-Inf, the whole update is skipped -- p, m, v and the bf16
 * copy keep every value -- LORA_FLAG_NONFINITE_GRAD is OR-ed into the
 * workspace status word, and the segment's skip flag (below) is 1; the caller
 * then keeps its step counter where it was.
 * Workspace: adam_workspace_bytes(n_seg) bytes (n_seg = 1 for adam_step).
 * Word 0 is the sticky status word (lora_device_status reads and clears it);
 * the int32 at byte offset 256 + 4 i is segment i's skip flag of the latest
 * call (1 = skipped, 0 = stepped), rewritten by every call.  Three launches:
 * clear the flags, scan g, update. */
size_t adam_workspace_bytes(int32_t n_seg);
lora_status adam_step(int64_t n, float* p, const float* g, float* m, float* v, int64_t step,
                      float lr, float beta1, float beta2, float eps, float weight_decay,
                      uint16_t* p_bf16, void* ws, size_t ws_bytes, void* stream);

/* Several adapters' AdamW steps in one set of launches: segment i updates
 * elements [offset, offset + count) of p, g, m, v (and p_bf16) exactly as
 * adam_step with step = segs[i].step would (same host-side bias factors, same
 * per-element arithmetic, so results are bitwise those of one adam_step call
 * per segment), and its skip decision is its own: a non-finite element in one
 * adapter's gradient skips that adapter only.  segs is a HOST array; segments
 * must not overlap.  Each adapter keeps its own step counter (OpenTinker,
 * "3 Approach": optimizer state local to each adapter).  n_seg >= 0. */
typedef struct { int64_t offset; int64_t count; int64_t step; } adam_segment;
lora_status adam_step_multi(int32_t n_seg, const adam_segment* segs, float* p, const float* g,
                            float* m, float* v, float lr, float beta1, float beta2, float eps,
                            float weight_decay, uint16_t* p_bf16, void* ws, size_t ws_bytes,
                            void* stream);

/* ---- MLP glue --------------------------------------------------------- */

/* SwiGLU between the gate/up and down projections: h = silu(g) * u, with
 * silu(z) = z / (1 + exp(-z)), in fp32, bf16 in and out.  n = element count. */
lora_status swiglu_forward(int64_t n, const uint16_t* gate, const uint16_t* up, uint16_t* h,
                           void* stream);
/* dg = dh * u * silu'(g), du = dh * silu(g). */
lora_status swiglu_backward(int64_t n, const uint16_t* dh, const uint16_t* gate,
                            const uint16_t* up, uint16_t* dgate, uint16_t* dup, void* stream);
/* out = a + b elementwise (bf16 in, fp32 sum, one round-to-nearest-even): the
 * MLP's dx is the sum of the gate and up projections' dx.  out may alias a or b. */
lora_status bf16_add(int64_t n, const uint16_t* a, const uint16_t* b, uint16_t* out,
                     void* stream);

/* ---- routed experts (mixture-of-experts layer) ------------------------ */

/* A top-k routed SwiGLU expert layer whose three projections (gate, up, down)
 * each carry the token's LoRA adapter on every expert (TPU RL note, section
 * 12 "Mixture-of-experts, and where adapters attach"; tinker-ticks "Step
 * time": the MoE pool touches every expert weight).  For token t with experts
 * e_1..e_K and weights w_1..w_K:
 *   y_t = sum_k w_k down_e(silu(gate_e x_t) * up_e x_t),
 *   proj_e(z) = W_e z + s B_{e,a} (A_{e,a} z),  a = adapter_ids[t].
 * Assignments j = t*K + k are sorted by the key e*(n_adapters + 1) + a; each
 * expert's rows run as one segment of a grouped GEMM and each (expert,
 * adapter) pair as one LoRA segment.  Routing weights are constants in the
 * backward (the router is not differentiated).
 * Layouts (bf16): W_gate, W_up [E][F][H]; W_down [E][H][F]; the backward takes
 * the per-expert transposes W_gate_t, W_up_t [E][H][F] and W_down_t [E][F][H]
 * (lora_transpose_bf16 per expert).  Descriptor tables are
 * [n_experts][n_adapters] per projection (gate/up: A [r][H], B [F][r]; down:
 * A [r][F], B [H][r]); an entry with rank 0 means "no adapter" for that pair.
 * A pair is active only when its entries are valid in all three tables
 * (otherwise LORA_FLAG_BAD_DESC and no LoRA for it).  Adapter ids out of range
 * give the base experts only (LORA_FLAG_ID_RANGE); an expert id out of range
 * drops that assignment (LORA_FLAG_ID_RANGE). */
typedef struct {
  int64_t n_tokens;        /* N */
  int64_t hidden;          /* H: multiple of 64 */
  int64_t d_ff;            /* F (expert intermediate): multiple of 64 */
  int64_t gate_pack_elems; /* pack sizes, for descriptor bounds checks */
  int64_t up_pack_elems;
  int64_t down_pack_elems;
  int32_t n_experts;       /* E: 1 .. 1024 */
  int32_t top_k;           /* K: 1 .. min(16, E); N*K < 2^30 */
  int32_t n_adapters;      /* E * (n_adapters + 1) <= 16384 */
  int32_t max_rank;        /* 16 .. 64, multiple of 16 */
} moe_shape;

/* Top-k routing of fp32 logits [n][n_experts]: experts int32 [n][top_k] by
 * descending logit (ties to the lower expert index; logits must be finite),
 * weights fp32 [n][top_k] = softmax over the chosen k (the full softmax
 * renormalised over its top k).  Expert ids are exact. */
lora_status moe_route(int64_t n, int32_t n_experts, int32_t top_k, const float* logits,
                      int32_t* experts, float* weights, void* stream);

/* Workspace for moe_forward / moe_backward, and the caller-owned buffer the
 * forward fills and the backward reads.  0 on an invalid shape.
 * "Position order": the assignments j = t*K + k stably sorted by key
 * e*(n_adapters + 1) + a (a = n_adapters for an adapter id out of range),
 * assignments with an expert id out of range last.  Saved layout, each region
 * starting at a multiple of 256 bytes in this order: gu (bf16 [N*K][2F] in
 * position order, each row the gate pre-activation then the up
 * pre-activation), h (bf16 [N*K][F], silu(gate)*up), then the scaled LoRA
 * vectors s*u of gate, up and down (bf16 hi/lo planes [2][N*K][max_rank]). */
size_t moe_workspace_bytes(const moe_shape* shape);
size_t moe_saved_bytes(const moe_shape* shape);

/*   x bf16 [N][H], experts int32 [N][K], weights fp32 [N][K], adapter_ids [N]
 *   y bf16 [N][H] out (fp32 weighted sum over the K experts, rounded once)
 *   saved: moe_saved_bytes bytes, 16-byte aligned, kept for moe_backward. */
lora_status moe_forward(const moe_shape* shape, const uint16_t* x, const int32_t* experts,
                        const float* weights, const int32_t* adapter_ids, const uint16_t* W_gate,
                        const uint16_t* W_up, const uint16_t* W_down, const uint16_t* gate_pack,
                        const uint16_t* up_pack, const uint16_t* down_pack,
                        const lora_adapter_desc* gate_desc, const lora_adapter_desc* up_desc,
                        const lora_adapter_desc* down_desc, uint16_t* y, void* saved, void* ws,
                        size_t ws_bytes, void* stream);

/*   dy bf16 [N][H]; dx bf16 [N][H] out; d*_pack fp32 gradient packs with the
 *   A/B packs' offsets: accumulate = 0 overwrites every active pair's region
 *   (zeros for pairs without assignments), != 0 adds into it.  Deterministic.
 *   trace (nullable): bf16 [3*N*K*F] out, the stage tensors in position
 *   order (for per-stage verification): dh [N*K][F], then [N*K][2F] rows of
 *   d(gate pre-activation) followed by d(up pre-activation). */
lora_status moe_backward(const moe_shape* shape, const uint16_t* dy, const uint16_t* x,
                         const int32_t* experts, const float* weights, const int32_t* adapter_ids,
                         const uint16_t* W_gate_t, const uint16_t* W_up_t,
                         const uint16_t* W_down_t, const uint16_t* gate_pack,
                         const uint16_t* up_pack, const uint16_t* down_pack,
                         const lora_adapter_desc* gate_desc, const lora_adapter_desc* up_desc,
                         const lora_adapter_desc* down_desc, const void* saved, uint16_t* dx,
                         float* dgate_pack, float* dup_pack, float* ddown_pack, int accumulate,
                         uint16_t* trace, void* ws, size_t ws_bytes, void* stream);

/* ---- SwiGLU MLP layer ------------------------------------------------ */

/* The dense SwiGLU MLP with the token's LoRA adapter on each of its three
 * projections (tinker-ticks, "How the SGMV kernel works": LoRA on every
 * linear layer, one batch mixing adapters; TPU RL note, section 12, for the
 * MLP's gate/up/down):
 *   y_t = down(silu(gate x_t) * up x_t),  proj(z) = W z + s B_a (A_a z).
 * It is the expert layer above with one expert and no routing: the same
 * kernels, the same saved layout ("position order" = tokens stably sorted by
 * adapter id, ids out of range last) and the same trace, with y and dx
 * written to token rows.  Layouts (bf16): W_gate, W_up [F][H]; W_down [H][F];
 * the backward takes W_gate_t, W_up_t [H][F] and W_down_t [F][H].  Descriptor
 * tables [n_adapters] per projection; a token whose adapter id is out of range
 * gets the base MLP only (LORA_FLAG_ID_RANGE); an adapter whose entry is
 * invalid in any table carries no LoRA (LORA_FLAG_BAD_DESC), rank 0 silently. */
typedef struct {
  int64_t n_tokens;        /* N < 2^30 */
  int64_t hidden;          /* H: multiple of 64 */
  int64_t d_ff;            /* F: multiple of 64 */
  int64_t gate_pack_elems; /* pack sizes, for descriptor bounds checks */
  int64_t up_pack_elems;
  int64_t down_pack_elems;
  int32_t n_adapters;      /* 1 .. 16383 */
  int32_t max_rank;        /* 16 .. 64, multiple of 16 */
} mlp_shape;

size_t mlp_workspace_bytes(const mlp_shape* shape);
size_t mlp_saved_bytes(const mlp_shape* shape);

/*   x bf16 [N][H], adapter_ids int32 [N]; y bf16 [N][H] out;
 *   saved: mlp_saved_bytes bytes, 16-byte aligned, kept for mlp_backward. */
lora_status mlp_forward(const mlp_shape* shape, const uint16_t* x, const int32_t* adapter_ids,
                        const uint16_t* W_gate, const uint16_t* W_up, const uint16_t* W_down,
                        const uint16_t* gate_pack, const uint16_t* up_pack,
                        const uint16_t* down_pack, const lora_adapter_desc* gate_desc,
                        const lora_adapter_desc* up_desc, const lora_adapter_desc* down_desc,
                        uint16_t* y, void* saved, void* ws, size_t ws_bytes, void* stream);

/*   dy bf16 [N][H]; dx bf16 [N][H] out; gradient packs and accumulate as for
 *   moe_backward; trace (nullable) as for moe_backward with N*K = N. */
lora_status mlp_backward(const mlp_shape* shape, const uint16_t* dy, const uint16_t* x,
                         const int32_t* adapter_ids, const uint16_t* W_gate_t,
                         const uint16_t* W_up_t, const uint16_t* W_down_t,
                         const uint16_t* gate_pack, const uint16_t* up_pack,
                         const uint16_t* down_pack, const lora_adapter_desc* gate_desc,
                         const lora_adapter_desc* up_desc, const lora_adapter_desc* down_desc,
                         const void* saved, uint16_t* dx, float* dgate_pack, float* dup_pack,
                         float* ddown_pack, int accumulate, uint16_t* trace, void* ws,
                         size_t ws_bytes, void* stream);

/* ---- forward without allocation ------------------------------------- */

/* For callers that cannot allocate device memory or hand in a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Computes exactly what lora_forward computes, with the same
 * kernels (same bits), but its scratch (segment tables, tile prefixes, status
 * word) is a fixed device array inside the library: lora_forward_noalloc_
 * scratch_bytes() = 2 MiB on each GPU the library runs on, held from the
 * library's load until the process ends.  Nothing is allocated on any path.
 *   status  int32 (device, nullable): this call's content flags (LORA_FLAG_*,
 *           as lora_forward would set in its workspace) are OR-ed into it.
 * A shape whose scratch exceeds the array (for example more than 65536
 * tokens with 1024 adapters) returns LORA_E_UNSUPPORTED before anything is
 * enqueued; other host errors as lora_forward.  The stream must belong to
 * the current device.  All calls on one GPU share that GPU's array and it
 * keeps the last call's contents: calls that overlap on one GPU (two streams
 * or two threads) race, so serialise them. */
size_t lora_forward_noalloc_scratch_bytes(void);
lora_status lora_forward_noalloc(const lora_shape* shape, const uint16_t* x, const uint16_t* W,
                                 const uint16_t* A_pack, const uint16_t* B_pack,
                                 const lora_adapter_desc* desc, const int32_t* adapter_ids,
                                 uint16_t* y, uint16_t* u_saved, int32_t* status, void* stream);

/* ---- measurement probes ----------------------------------------------- */

/* The chip's own peaks, for reporting the kernels' fractions against measured
 * as well as published figures.  lora_probe_mfma runs `blocks` blocks of 8
 * waves, each wave `iters` rounds of 4 independent v_mfma_f32_32x32x16_bf16
 * on register operands (no memory traffic); its flop count is
 * lora_probe_mfma_flops_per_iter(blocks) * iters.  sink: device float[blocks]
 * (written, meaningless).  lora_probe_copy copies `bytes` (a multiple of 16,
 * 16-byte aligned buffers) with a streaming kernel: 2 * bytes of HBM traffic.
 * lora_probe_read streams `bytes` of src through the chip (reads only; sink:
 * one device uint32, almost never written). */
int64_t lora_probe_mfma_flops_per_iter(int32_t blocks);
lora_status lora_probe_mfma(int64_t iters, int32_t blocks, float* sink, void* stream);
lora_status lora_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);
lora_status lora_probe_read(const void* src, int64_t bytes, void* sink, void* stream);

/* ---- kernel timing (measurement) ------------------------------------- */

/* When enabled, the library brackets each launch of the kernel classes below
 * with HIP events on the launch stream.  lora_timing_read synchronises on the
 * recorded events and returns the summed duration (ms) and launch count since
 * the last reset.  The timers are per host thread (enable, reset and read on
 * the thread that makes the calls); off by default. */
#define LORA_TIMER_BASE_GEMM     0   /* y = x W^T and dx = dy W GEMMs */
#define LORA_TIMER_LOGPROB_FWD   1   /* lm_head GEMM with online logsumexp */
#define LORA_TIMER_LOGPROB_BWD   2   /* logit recompute + dh GEMMs */
#define LORA_TIMER_SHRINK        3
#define LORA_TIMER_EXPAND        4   /* reserved: the expand runs inside the base GEMMs */
#define LORA_TIMER_GRAD          5   /* dA / dB reductions */
#define LORA_TIMER_ADAM          6
#define LORA_TIMER_COUNT         7
void lora_timing_enable(int on);
void lora_timing_reset(void);
lora_status lora_timing_read(int32_t timer, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* LORA_MI355X_H */
