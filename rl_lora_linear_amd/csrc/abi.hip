// C-ABI entry points: host-side validation, workspace carving and the launch
// sequence of each call.  All work is enqueued on the caller's stream.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"
#include "segments.hpp"
#include "sgmv.hpp"

// ------------------------------------------------------------------ errors
namespace lora_host {

static thread_local std::string g_err;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
}

lora_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return LORA_OK;
  set_error("%s: %s", what, hipGetErrorString(e));
  return LORA_E_HIP;
}

lora_status launch_check(const char* what) { return hip_check(hipGetLastError(), what); }

int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// ------------------------------------------------------------------ timing
// Measurement hooks, per host thread: each thread that enables timing keeps its
// own event pairs (created on first use, kept until the process ends), so the
// calls stay free of shared mutable state.
struct TimerState {
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pairs[LORA_TIMER_COUNT];
  size_t used[LORA_TIMER_COUNT] = {};
};
static thread_local TimerState g_tim;

void timer_begin(int timer, hipStream_t s) {
  if (!g_tim.on) return;
  auto& v = g_tim.pairs[timer];
  size_t& u = g_tim.used[timer];
  if (u == v.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return;
    v.emplace_back(a, b);
  }
  (void)hipEventRecord(v[u].first, s);
}

void timer_end(int timer, hipStream_t s) {
  if (!g_tim.on) return;
  auto& v = g_tim.pairs[timer];
  size_t& u = g_tim.used[timer];
  if (u >= v.size()) return;
  (void)hipEventRecord(v[u].second, s);
  ++u;
}

}  // namespace lora_host

using namespace lora_host;
using lora::cdiv;

static inline hipStream_t S(void* p) { return (hipStream_t)p; }

#define TRY(expr)                  \
  do {                             \
    lora_status _st = (expr);      \
    if (_st != LORA_OK) return _st; \
  } while (0)

// ------------------------------------------------------------------ layer workspace
namespace {

constexpr int kTmShrink = 32;       // rows per shrink tile (matches the kernel)
constexpr int kTmShrinkTall = 128;  // rows per tall shrink tile (large batches)

struct LayerWs {
  char* seg;          // status word + segment scratch
  size_t seg_bytes;
  int32_t* perm;
  int32_t* adpos;     // adapter of each segment position (-1: none)
  int32_t* offsets;
  uint8_t* active;
  int32_t* pre32;
  int32_t* pre128;
  int32_t* prec;
  uint16_t* v;        // scaled v = s_a B_a^T dy as bf16 hi/lo planes [2][N][max_rank]
  uint16_t* zero;     // 256 zero bytes (source of the rows past a gradient chunk)
  float* partial;     // dB chunk partials
  float* partial_a;   // dA chunk partials
  float* shpart;      // chunk sums of a K-split shrink (null: the shrinks do not split)
  size_t shpart_floats;
  size_t total;
};

// fwd_only: the forward's part alone (no v planes, no gradient partials, no
// K-split shrink buffer: its shrink runs unsplit, with the same bits)
LayerWs carve_layer(const lora_shape& sh, void* ws, size_t bytes, bool fwd_only = false) {
  Carve cv(ws, bytes);
  LayerWs w{};
  w.seg_bytes = segments_ws_bytes(sh.n_tokens, sh.n_adapters);
  w.seg = cv.take<char>(w.seg_bytes);
  w.perm = cv.take<int32_t>((size_t)std::max<int64_t>(sh.n_tokens, 1));
  w.adpos = cv.take<int32_t>((size_t)std::max<int64_t>(sh.n_tokens, 1));
  w.offsets = cv.take<int32_t>((size_t)sh.n_adapters + 1);
  w.active = cv.take<uint8_t>((size_t)sh.n_adapters);
  w.pre32 = cv.take<int32_t>((size_t)sh.n_adapters + 1);
  w.pre128 = cv.take<int32_t>((size_t)sh.n_adapters + 1);
  w.prec = cv.take<int32_t>((size_t)sh.n_adapters + 1);
  w.zero = cv.take<uint16_t>(128);
  if (fwd_only) {
    w.v = nullptr;
    w.total = cv.used;
    return w;
  }
  w.v = cv.take<uint16_t>((size_t)2 * std::max<int64_t>(sh.n_tokens, 1) * sh.max_rank);
  // chunk partials of dB and of dA (reduced in one launch, so apart)
  w.partial = cv.take<float>((size_t)grad_partial_floats(sh.n_tokens, sh.n_adapters, sh.d_out,
                                                         sh.max_rank));
  w.partial_a = cv.take<float>((size_t)grad_partial_floats(sh.n_tokens, sh.n_adapters, sh.d_in,
                                                           sh.max_rank));
  w.shpart_floats = std::max(shrink_part_floats(sh.n_tokens, sh.n_adapters, (int)sh.d_in),
                             shrink_part_floats(sh.n_tokens, sh.n_adapters, (int)sh.d_out));
  w.shpart = w.shpart_floats ? cv.take<float>(w.shpart_floats) : nullptr;
  w.total = cv.used;
  return w;
}

lora_status check_shape(const lora_shape* sh) {
  LORA_ARG_CHECK(sh != nullptr, "shape is NULL");
  LORA_ARG_CHECK(sh->n_tokens >= 0 && sh->n_tokens <= INT32_MAX / 2,
                 "n_tokens %lld outside [0, 2^30)", (long long)sh->n_tokens);
  LORA_ARG_CHECK(sh->d_in > 0 && sh->d_out > 0, "d_in and d_out must be positive");
  LORA_ARG_CHECK(sh->n_adapters >= 1 && sh->n_adapters <= 16384, "n_adapters %d outside [1, 16384]",
                 sh->n_adapters);
  LORA_ARG_CHECK(sh->max_rank >= 16 && sh->max_rank <= 64 && sh->max_rank % 16 == 0,
                 "max_rank %d must be a multiple of 16 in [16, 64]", sh->max_rank);
  LORA_ARG_CHECK(sh->order == LORA_IDS_SORTED || sh->order == LORA_IDS_INTERLEAVED,
                 "order %d is not a lora_id_order", sh->order);
  LORA_ARG_CHECK(sh->reserved == 0, "reserved field must be 0");
  LORA_ARG_CHECK(sh->a_pack_elems >= 0 && sh->b_pack_elems >= 0, "pack sizes must be >= 0");
  if (sh->d_in % 64 || sh->d_out % 64 || sh->d_in > (1 << 20) || sh->d_out > (1 << 20)) {
    set_error("d_in %lld and d_out %lld must be multiples of 64 and <= 2^20",
              (long long)sh->d_in, (long long)sh->d_out);
    return LORA_E_UNSUPPORTED;
  }
  return LORA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

lora_status layer_segments(const lora_shape& sh, const lora_adapter_desc* desc,
                           const int32_t* ids, const LayerWs& w, hipStream_t s) {
  SegExtras ex{};
  ex.tab[0] = SegDescs{desc, sh.d_in, sh.d_out, sh.a_pack_elems, sh.b_pack_elems};
  ex.n_tabs = 1;
  ex.max_rank = sh.max_rank;
  ex.active = w.active;
  ex.tm[0] = kTmShrink;
  ex.pre[0] = w.pre32;
  ex.tm[1] = kTmShrinkTall;
  ex.pre[1] = w.pre128;
  ex.tm[2] = kGradChunk;
  ex.pre[2] = w.prec;
  ex.adpos = w.adpos;
  return run_segments(ids, sh.n_tokens, sh.n_adapters, sh.order, w.perm, w.offsets, &ex, w.seg,
                      w.seg_bytes, s);
}

}  // namespace

extern "C" {

size_t lora_workspace_bytes(const lora_shape* shape) {
  if (check_shape(shape) != LORA_OK) return 0;
  return carve_layer(*shape, nullptr, 0).total;
}

lora_status lora_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes < 256) {
    set_error("workspace NULL or smaller than 256 bytes");
    return LORA_E_WORKSPACE;
  }
  return launch_fill_i32((int32_t*)ws, 64, 0, S(stream));
}

lora_status lora_device_status(void* ws, int32_t* host_flags, void* stream) {
  LORA_ARG_CHECK(ws != nullptr && host_flags != nullptr, "NULL workspace or flags pointer");
  TRY(hip_check(hipStreamSynchronize(S(stream)), "hipStreamSynchronize"));
  int32_t v = 0;
  TRY(hip_check(hipMemcpy(&v, ws, sizeof(v), hipMemcpyDeviceToHost), "status read"));
  const int32_t z = 0;
  TRY(hip_check(hipMemcpy(ws, &z, sizeof(z), hipMemcpyHostToDevice), "status clear"));
  *host_flags = v;
  if (v) {
    set_error("device content checks failed: flags 0x%x", v);
    return LORA_E_DEVICE_CHECK;
  }
  return LORA_OK;
}

const char* lora_last_error(void) { return g_err.c_str(); }

size_t lora_segments_workspace_bytes(int64_t n, int32_t n_keys) {
  if (n < 0 || n_keys < 1 || n_keys > 16384) return 0;
  return segments_ws_bytes(n, n_keys);
}

lora_status lora_segments(const int32_t* ids, int64_t n, int32_t n_keys, int32_t order,
                          int32_t* perm, int32_t* offsets, void* ws, size_t ws_bytes,
                          void* stream) {
  LORA_ARG_CHECK(n >= 0 && n <= INT32_MAX / 2, "n %lld outside [0, 2^30)", (long long)n);
  LORA_ARG_CHECK(n_keys >= 1 && n_keys <= 16384, "n_keys %d outside [1, 16384]", n_keys);
  LORA_ARG_CHECK(order == LORA_IDS_SORTED || order == LORA_IDS_INTERLEAVED, "bad order %d", order);
  LORA_ARG_CHECK(offsets != nullptr, "offsets is NULL");
  LORA_ARG_CHECK(n == 0 || (ids != nullptr && perm != nullptr), "ids/perm NULL");
  if (!ws || ws_bytes < segments_ws_bytes(n, n_keys)) {
    set_error("segments: workspace too small (%zu < %zu)", ws_bytes, segments_ws_bytes(n, n_keys));
    return LORA_E_WORKSPACE;
  }
  return run_segments(ids, n, n_keys, order, perm, offsets, nullptr, ws, ws_bytes, S(stream));
}

lora_status lora_transpose_bf16(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t cols,
                                void* stream) {
  LORA_ARG_CHECK(src && dst && src != dst, "src/dst NULL or equal");
  LORA_ARG_CHECK(rows > 0 && cols > 0, "rows and cols must be positive");
  if (rows % 64 || cols % 64) {
    set_error("transpose: rows %lld and cols %lld must be multiples of 64", (long long)rows,
              (long long)cols);
    return LORA_E_UNSUPPORTED;
  }
  return launch_transpose_bf16(src, dst, rows, cols, S(stream));
}

static lora_status forward_checks(const lora_shape* shape, const uint16_t* x, const uint16_t* W,
                                  const uint16_t* A_pack, const uint16_t* B_pack,
                                  const lora_adapter_desc* desc, const int32_t* adapter_ids,
                                  uint16_t* y, uint16_t* u_saved) {
  TRY(check_shape(shape));
  const lora_shape& sh = *shape;
  LORA_ARG_CHECK(W && A_pack && B_pack && desc, "W, A_pack, B_pack and desc must be non-NULL");
  LORA_ARG_CHECK(sh.n_tokens == 0 || (x && adapter_ids && y && u_saved),
                 "x, adapter_ids, y and u_saved must be non-NULL");
  LORA_ARG_CHECK(sh.n_tokens == 0 || (aligned16(x) && aligned16(y) && aligned16(u_saved)),
                 "x, y and u_saved must be 16-byte aligned");
  LORA_ARG_CHECK(aligned16(W) && aligned16(A_pack) && aligned16(B_pack), "W and the packs must be 16-byte aligned");
  return LORA_OK;
}

// The forward's launches on a carved workspace (segments, shrink, GEMM with the
// fused expand); every part of `w` it reads it has written earlier in the call,
// except the sticky status word.
static lora_status forward_core(const lora_shape& sh, const uint16_t* x, const uint16_t* W,
                                const uint16_t* A_pack, const uint16_t* B_pack,
                                const lora_adapter_desc* desc, const int32_t* adapter_ids,
                                uint16_t* y, uint16_t* u_saved, const LayerWs& w, hipStream_t s) {
  const int N = (int)sh.n_tokens;
  TRY(layer_segments(sh, desc, adapter_ids, w, s));
  if (N == 0) return LORA_OK;
  timer_begin(LORA_TIMER_SHRINK, s);
  TRY(launch_shrink(x, sh.d_in, (int)sh.d_in, A_pack, 0, desc, w.adpos, w.perm, w.perm, nullptr,
                    w.offsets, w.pre32, sh.n_adapters, sh.n_tokens, u_saved, sh.max_rank, w.zero,
                    s, nullptr, nullptr, nullptr, w.pre128, w.shpart, w.shpart_floats));
  timer_end(LORA_TIMER_SHRINK, s);
  // base GEMM over rows in segment order with the expand y += B_a (s u) fused
  GemmRows f;
  f.a_rows = f.c_rows = w.perm;
  f.a_rows_bound = sh.n_tokens;
  f.vec = u_saved;
  f.vec_plane = sh.n_tokens * sh.max_rank;
  f.vec_ld = sh.max_rank;
  f.use_b_off = 1;
  f.lmat = B_pack;
  f.desc = desc;
  f.adpos = w.adpos;
  f.n_ad = sh.n_adapters;
  timer_begin(LORA_TIMER_BASE_GEMM, s);
  TRY(gemm_nt_rows(x, W, y, N, (int)sh.d_out, (int)sh.d_in, sh.d_in, sh.d_in, sh.d_out, f, s));
  timer_end(LORA_TIMER_BASE_GEMM, s);
  return LORA_OK;
}

lora_status lora_forward(const lora_shape* shape, const uint16_t* x, const uint16_t* W,
                         const uint16_t* A_pack, const uint16_t* B_pack,
                         const lora_adapter_desc* desc, const int32_t* adapter_ids, uint16_t* y,
                         uint16_t* u_saved, void* ws, size_t ws_bytes, void* stream) {
  TRY(forward_checks(shape, x, W, A_pack, B_pack, desc, adapter_ids, y, u_saved));
  LayerWs w = carve_layer(*shape, ws, ws_bytes);
  if (!ws || w.total > ws_bytes) {
    set_error("lora_forward: workspace %zu bytes < %zu needed", ws_bytes, w.total);
    return LORA_E_WORKSPACE;
  }
  return forward_core(*shape, x, W, A_pack, B_pack, desc, adapter_ids, y, u_saved, w, S(stream));
}

lora_status lora_backward(const lora_shape* shape, const uint16_t* dy, const uint16_t* x,
                          const uint16_t* W_t, const uint16_t* A_pack, const uint16_t* B_pack,
                          const lora_adapter_desc* desc, const int32_t* adapter_ids,
                          const uint16_t* u_saved, uint16_t* dx, float* dA_pack, float* dB_pack,
                          int accumulate, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_shape(shape));
  const lora_shape& sh = *shape;
  LORA_ARG_CHECK(W_t && A_pack && B_pack && desc && dA_pack && dB_pack,
                 "W_t, packs, desc and gradient packs must be non-NULL");
  LORA_ARG_CHECK(sh.n_tokens == 0 || (dy && x && adapter_ids && u_saved && dx),
                 "dy, x, adapter_ids, u_saved and dx must be non-NULL");
  LORA_ARG_CHECK(sh.n_tokens == 0 || (aligned16(dy) && aligned16(x) && aligned16(dx) && aligned16(u_saved)),
                 "dy, x, dx and u_saved must be 16-byte aligned");
  LORA_ARG_CHECK(aligned16(W_t) && aligned16(A_pack) && aligned16(B_pack) && aligned16(dA_pack) &&
                     aligned16(dB_pack),
                 "W_t and the packs must be 16-byte aligned");
  LayerWs w = carve_layer(sh, ws, ws_bytes);
  if (!ws || w.total > ws_bytes) {
    set_error("lora_backward: workspace %zu bytes < %zu needed", ws_bytes, w.total);
    return LORA_E_WORKSPACE;
  }
  hipStream_t s = S(stream);
  const int N = (int)sh.n_tokens;
  TRY(layer_segments(sh, desc, adapter_ids, w, s));
  if (N > 0) {
    timer_begin(LORA_TIMER_SHRINK, s);
    TRY(launch_shrink(dy, sh.d_out, (int)sh.d_out, B_pack, 1, desc, w.adpos, w.perm, w.perm,
                      nullptr, w.offsets, w.pre32, sh.n_adapters, sh.n_tokens, w.v, sh.max_rank,
                      w.zero, s, nullptr, nullptr, nullptr, w.pre128, w.shpart, w.shpart_floats));
    timer_end(LORA_TIMER_SHRINK, s);
    // dX = dY W over rows in segment order with the expand dX += A_a^T (s v) fused
    GemmRows f;
    f.a_rows = f.c_rows = w.perm;
    f.a_rows_bound = sh.n_tokens;
    f.vec = w.v;
    f.vec_plane = sh.n_tokens * sh.max_rank;
    f.vec_ld = sh.max_rank;
    f.use_b_off = 0;
    f.lmat_ld = sh.d_in;
    f.lmat = A_pack;
    f.desc = desc;
    f.adpos = w.adpos;
    f.n_ad = sh.n_adapters;
    timer_begin(LORA_TIMER_BASE_GEMM, s);
    TRY(gemm_nt_rows(dy, W_t, dx, N, (int)sh.d_in, (int)sh.d_out, sh.d_out, sh.d_out, sh.d_in, f, s));
    timer_end(LORA_TIMER_BASE_GEMM, s);
  }
  timer_begin(LORA_TIMER_GRAD, s);
  // dB = s sum dy u^T and dA = s sum v x^T over each adapter's tokens, one launch
  TRY(launch_grad_pair(u_saved, dy, sh.d_out, (int)sh.d_out, dB_pack, w.partial, w.v, x, sh.d_in,
                       (int)sh.d_in, dA_pack, w.partial_a, sh.max_rank, w.zero, desc, w.active,
                       w.perm, w.offsets, w.prec, sh.n_adapters, sh.n_tokens, accumulate, s));
  timer_end(LORA_TIMER_GRAD, s);
  return LORA_OK;
}

// ------------------------------------------------------------------ logprobs
static size_t logprob_ws(int64_t n, int64_t vocab, float** pm, float** ps, float** zt, void* ws,
                         size_t bytes) {
  Carve cv(ws, bytes);
  cv.take<int32_t>(64);
  const int64_t tiles = cdiv(vocab, 256);
  float* a = cv.take<float>((size_t)tiles * std::max<int64_t>(n, 1));
  float* b = cv.take<float>((size_t)tiles * std::max<int64_t>(n, 1));
  float* c = cv.take<float>((size_t)std::max<int64_t>(n, 1));
  if (pm) { *pm = a; *ps = b; *zt = c; }
  return cv.used;
}

// The size queries accept exactly the n and vocab the entry points accept
// (check_lp below) and return 0 for anything else.
static bool lp_sizes_ok(int64_t n, int64_t vocab) {
  return n >= 0 && n <= INT32_MAX / 2 && vocab > 0 && vocab % 64 == 0 && vocab <= INT32_MAX / 2;
}

size_t token_logprobs_workspace_bytes(int64_t n, int64_t vocab) {
  if (!lp_sizes_ok(n, vocab)) return 0;
  return logprob_ws(n, vocab, nullptr, nullptr, nullptr, nullptr, 0);
}

static lora_status check_lp(int64_t n, int64_t hidden, int64_t vocab) {
  LORA_ARG_CHECK(n >= 0 && n <= INT32_MAX / 2, "n %lld outside [0, 2^30)", (long long)n);
  LORA_ARG_CHECK(hidden > 0 && vocab > 0, "hidden and vocab must be positive");
  if (hidden % 64 || vocab % 64 || vocab > INT32_MAX / 2 || hidden > (1 << 20)) {
    set_error("hidden %lld and vocab %lld must be multiples of 64", (long long)hidden, (long long)vocab);
    return LORA_E_UNSUPPORTED;
  }
  return LORA_OK;
}

lora_status token_logprobs(int64_t n, int64_t hidden, int64_t vocab, const uint16_t* h,
                           const uint16_t* lm_head, const int32_t* targets, float* logprobs,
                           float* lse, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_lp(n, hidden, vocab));
  LORA_ARG_CHECK(lm_head != nullptr, "lm_head is NULL");
  LORA_ARG_CHECK(n == 0 || (h && targets && logprobs && lse), "h/targets/logprobs/lse NULL");
  LORA_ARG_CHECK(aligned16(lm_head) && (n == 0 || aligned16(h)), "h and lm_head must be 16-byte aligned");
  float *pm, *ps, *zt;
  const size_t need = logprob_ws(n, vocab, &pm, &ps, &zt, ws, ws_bytes);
  if (!ws || need > ws_bytes) {
    set_error("token_logprobs: workspace %zu bytes < %zu needed", ws_bytes, need);
    return LORA_E_WORKSPACE;
  }
  if (n == 0) return LORA_OK;
  hipStream_t s = S(stream);
  timer_begin(LORA_TIMER_LOGPROB_FWD, s);
  TRY(gemm_nt_lse(h, lm_head, (int)n, (int)vocab, (int)hidden, hidden, hidden, pm, ps, zt, targets, s));
  timer_end(LORA_TIMER_LOGPROB_FWD, s);
  return launch_logprob_merge(pm, ps, zt, targets, n, (int)cdiv(vocab, 256), vocab, logprobs, lse,
                              (int32_t*)ws, s);
}

size_t token_logprobs_backward_workspace_bytes(int64_t n, int64_t vocab, int64_t chunk_rows) {
  if (!lp_sizes_ok(n, vocab) || chunk_rows < 256) return 0;
  // The entry point never runs a chunk longer than n rounded up to 256 rows.
  const int64_t rows = std::min(lora::align_up(std::min<int64_t>(chunk_rows, INT32_MAX / 2), 256),
                                lora::align_up(std::max<int64_t>(n, 1), 256));
  Carve cv(nullptr, 0);
  cv.take<int32_t>(64);
  cv.take<uint16_t>((size_t)rows * vocab);
  return cv.used;
}

lora_status token_logprobs_backward(int64_t n, int64_t hidden, int64_t vocab, const uint16_t* h,
                                    const uint16_t* lm_head, const uint16_t* lm_head_t,
                                    const int32_t* targets, const float* lse, const float* dlogp,
                                    uint16_t* dh, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_lp(n, hidden, vocab));
  LORA_ARG_CHECK(lm_head && lm_head_t, "lm_head and lm_head_t must be non-NULL");
  LORA_ARG_CHECK(n == 0 || (h && targets && lse && dlogp && dh), "h/targets/lse/dlogp/dh NULL");
  LORA_ARG_CHECK(aligned16(lm_head) && aligned16(lm_head_t) && (n == 0 || (aligned16(h) && aligned16(dh))),
                 "h, dh and the lm_head copies must be 16-byte aligned");
  const size_t head = 256;
  if (!ws || ws_bytes < head + (size_t)256 * vocab * 2) {
    set_error("token_logprobs_backward: workspace must hold at least 256 rows of G (%zu bytes)",
              head + (size_t)256 * vocab * 2);
    return LORA_E_WORKSPACE;
  }
  int64_t chunk = (int64_t)((ws_bytes - head) / ((size_t)vocab * 2));
  chunk = (chunk / 256) * 256;
  if (chunk > lora::align_up(n, 256)) chunk = lora::align_up(n, 256);
  uint16_t* G = (uint16_t*)((char*)ws + head);
  hipStream_t s = S(stream);
  for (int64_t c0 = 0; c0 < n; c0 += chunk) {
    const int rows = (int)std::min<int64_t>(chunk, n - c0);
    timer_begin(LORA_TIMER_LOGPROB_BWD, s);
    TRY(gemm_nt_grad(h + c0 * hidden, lm_head, G, vocab, rows, (int)vocab, (int)hidden, hidden,
                     hidden, targets + c0, lse + c0, dlogp + c0, s));
    TRY(gemm_nt_bf16(G, lm_head_t, dh + c0 * hidden, rows, (int)hidden, (int)vocab, vocab, vocab,
                     hidden, s));
    timer_end(LORA_TIMER_LOGPROB_BWD, s);
  }
  return LORA_OK;
}

// ------------------------------------------------------------------ loss
size_t loss_grad_workspace_bytes(int64_t n) {
  if (n < 0 || n > INT32_MAX / 2) return 0;
  return 256 + (size_t)std::max<int64_t>(1, cdiv(n, 1024)) * sizeof(double);
}

lora_status loss_grad(int32_t kind, int64_t n, const float* logprobs, const float* weights,
                      const float* advantages, const float* sampler_logprobs,
                      const float* custom_g, const loss_config* cfg, float* loss_out,
                      float* dlogp, void* ws, size_t ws_bytes, void* stream) {
  LORA_ARG_CHECK(kind >= LOSS_CROSS_ENTROPY && kind <= LOSS_CUSTOM, "unknown loss kind %d", kind);
  LORA_ARG_CHECK(n >= 0 && n <= INT32_MAX / 2, "n %lld outside [0, 2^30)", (long long)n);
  LORA_ARG_CHECK(loss_out != nullptr, "loss_out is NULL");
  LORA_ARG_CHECK(n == 0 || (logprobs && weights && dlogp), "logprobs/weights/dlogp NULL");
  if (kind == LOSS_IMPORTANCE_SAMPLING || kind == LOSS_PPO)
    LORA_ARG_CHECK(n == 0 || (advantages && sampler_logprobs), "advantages and sampler_logprobs required");
  if (kind == LOSS_CUSTOM) LORA_ARG_CHECK(n == 0 || custom_g, "custom_g required");
  float lo = 0.2f, hi = 0.2f;
  if (kind == LOSS_PPO) {
    LORA_ARG_CHECK(cfg != nullptr, "ppo needs a loss_config");
    LORA_ARG_CHECK(cfg->clip_low >= 0.f && cfg->clip_low < 1.f && cfg->clip_high >= 0.f,
                   "clip bounds need 0 <= clip_low < 1 and clip_high >= 0");
    lo = cfg->clip_low;
    hi = cfg->clip_high;
  }
  if (!ws || ws_bytes < loss_grad_workspace_bytes(n)) {
    set_error("loss_grad: workspace too small");
    return LORA_E_WORKSPACE;
  }
  return launch_loss(kind, n, logprobs, weights, advantages, sampler_logprobs, custom_g, lo, hi,
                     (double*)((char*)ws + 256), loss_out, dlogp, (int32_t*)ws, S(stream));
}

// ------------------------------------------------------------------ Adam
size_t adam_workspace_bytes(int32_t n_seg) {
  if (n_seg < 0) return 0;
  return 256 + (size_t)lora::align_up(std::max<int64_t>(1, n_seg) * 4, 256);
}

static lora_status adam_run(int32_t n_seg, const int64_t* off, const int64_t* cnt,
                            const int64_t* step, float* p, const float* g, float* m, float* v,
                            float lr, float beta1, float beta2, float eps, float weight_decay,
                            uint16_t* p_bf16, void* ws, size_t ws_bytes, hipStream_t s) {
  LORA_ARG_CHECK(beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f, "betas must lie in [0, 1)");
  std::vector<float> ss(n_seg), ib(n_seg);
  for (int i = 0; i < n_seg; ++i) {
    LORA_ARG_CHECK(off[i] >= 0 && cnt[i] >= 0, "segment %d: negative offset/count", i);
    LORA_ARG_CHECK(step[i] >= 1, "segment %d: step must be >= 1 (1-based per-adapter counter)", i);
    const double bc1 = 1.0 - std::pow((double)beta1, (double)step[i]);
    const double bc2 = 1.0 - std::pow((double)beta2, (double)step[i]);
    ss[i] = (float)((double)lr / bc1);
    ib[i] = (float)(1.0 / std::sqrt(bc2));
  }
  if (!ws || ws_bytes < adam_workspace_bytes(n_seg)) {
    set_error("adam: workspace too small (need adam_workspace_bytes(%d))", n_seg);
    return LORA_E_WORKSPACE;
  }
  if (n_seg == 0) return LORA_OK;
  timer_begin(LORA_TIMER_ADAM, s);
  TRY(launch_adam_multi(n_seg, off, cnt, ss.data(), ib.data(), p, g, m, v, lr, beta1, beta2, eps,
                        weight_decay, p_bf16, (int32_t*)((char*)ws + 256), (int32_t*)ws, s));
  timer_end(LORA_TIMER_ADAM, s);
  return LORA_OK;
}

lora_status adam_step(int64_t n, float* p, const float* g, float* m, float* v, int64_t step,
                      float lr, float beta1, float beta2, float eps, float weight_decay,
                      uint16_t* p_bf16, void* ws, size_t ws_bytes, void* stream) {
  LORA_ARG_CHECK(n >= 0, "n must be >= 0");
  LORA_ARG_CHECK(n == 0 || (p && g && m && v), "p/g/m/v NULL");
  const int64_t off = 0;
  return adam_run(1, &off, &n, &step, p, g, m, v, lr, beta1, beta2, eps, weight_decay, p_bf16, ws,
                  ws_bytes, S(stream));
}

lora_status adam_step_multi(int32_t n_seg, const adam_segment* segs, float* p, const float* g,
                            float* m, float* v, float lr, float beta1, float beta2, float eps,
                            float weight_decay, uint16_t* p_bf16, void* ws, size_t ws_bytes,
                            void* stream) {
  LORA_ARG_CHECK(n_seg >= 0, "n_seg must be >= 0");
  if (n_seg == 0) return LORA_OK;
  LORA_ARG_CHECK(segs != nullptr, "segs is NULL");
  LORA_ARG_CHECK(p && g && m && v, "p/g/m/v NULL");
  std::vector<int64_t> off(n_seg), cnt(n_seg), step(n_seg);
  for (int i = 0; i < n_seg; ++i) {
    off[i] = segs[i].offset;
    cnt[i] = segs[i].count;
    step[i] = segs[i].step;
  }
  return adam_run(n_seg, off.data(), cnt.data(), step.data(), p, g, m, v, lr, beta1, beta2, eps,
                  weight_decay, p_bf16, ws, ws_bytes, S(stream));
}

// ------------------------------------------------------------------ SwiGLU
lora_status swiglu_forward(int64_t n, const uint16_t* gate, const uint16_t* up, uint16_t* h,
                           void* stream) {
  LORA_ARG_CHECK(n >= 0 && (n == 0 || (gate && up && h)), "bad swiglu_forward arguments");
  LORA_ARG_CHECK(n == 0 || (aligned16(gate) && aligned16(up) && aligned16(h)), "swiglu buffers must be 16-byte aligned");
  return launch_swiglu_fwd(n, gate, up, h, S(stream));
}

lora_status swiglu_backward(int64_t n, const uint16_t* dh, const uint16_t* gate,
                            const uint16_t* up, uint16_t* dgate, uint16_t* dup, void* stream) {
  LORA_ARG_CHECK(n >= 0 && (n == 0 || (dh && gate && up && dgate && dup)), "bad swiglu_backward arguments");
  LORA_ARG_CHECK(n == 0 || (aligned16(dh) && aligned16(gate) && aligned16(up) && aligned16(dgate) && aligned16(dup)),
                 "swiglu buffers must be 16-byte aligned");
  return launch_swiglu_bwd(n, dh, gate, up, dgate, dup, S(stream));
}

}  // extern "C"

// ------------------------------------------------------------------ MoE
static lora_status check_moe(const moe_shape* sh) {
  LORA_ARG_CHECK(sh != nullptr, "moe shape is NULL");
  LORA_ARG_CHECK(sh->n_tokens >= 0 && sh->n_tokens * sh->top_k <= INT32_MAX / 2,
                 "n_tokens * top_k must be < 2^30");
  LORA_ARG_CHECK(sh->n_experts >= 1 && sh->n_experts <= 1024, "n_experts %d outside [1, 1024]",
                 sh->n_experts);
  LORA_ARG_CHECK(sh->top_k >= 1 && sh->top_k <= 16 && sh->top_k <= sh->n_experts,
                 "top_k %d outside [1, min(16, n_experts)]", sh->top_k);
  LORA_ARG_CHECK(sh->n_adapters >= 1 && (int64_t)sh->n_experts * (sh->n_adapters + 1) <= 16384,
                 "n_adapters %d: n_experts * (n_adapters + 1) must be <= 16384", sh->n_adapters);
  LORA_ARG_CHECK(sh->max_rank >= 16 && sh->max_rank <= 64 && sh->max_rank % 16 == 0,
                 "max_rank %d must be a multiple of 16 in [16, 64]", sh->max_rank);
  LORA_ARG_CHECK(sh->gate_pack_elems >= 0 && sh->up_pack_elems >= 0 && sh->down_pack_elems >= 0,
                 "pack sizes must be >= 0");
  if (sh->hidden <= 0 || sh->d_ff <= 0 || sh->hidden % 64 || sh->d_ff % 64 ||
      sh->hidden > (1 << 20) || sh->d_ff > (1 << 20)) {
    set_error("hidden %lld and d_ff %lld must be positive multiples of 64 and <= 2^20",
              (long long)sh->hidden, (long long)sh->d_ff);
    return LORA_E_UNSUPPORTED;
  }
  return LORA_OK;
}

namespace {

// Assignments j = t*K + k sorted by key e*(n_ad + 1) + a ("position" order).
struct MoeWs {
  char* seg;
  size_t seg_bytes;
  int32_t* keys;     // [NK]
  int32_t* perm;     // position -> assignment
  int32_t* adpos;    // position -> key (-1: none)
  int32_t* tokrow;   // position -> token
  int32_t* inv;      // assignment -> position
  int32_t* offsets;  // [n_keys + 1]
  uint8_t* active;   // [n_keys]
  int32_t* pre32;
  int32_t* pre128;
  int32_t* prec;
  int32_t* gpre;     // [E + 1]
  lora_adapter_desc* desc[3];  // per-key tables (gate, up, down) with "no adapter" entries
  uint16_t* zero;
  uint16_t* o;       // forward: expert outputs [NK][H] bf16
  float* wpos;       // backward: routing weight per position
  uint16_t* v[3];    // backward: s*v planes per projection [2][NK][R] (down: s*w*v)
  uint16_t* uw;      // backward: w * (s u_down) planes
  uint16_t* dh;      // [NK][F] (the trace's, else not stored)
  uint16_t* dgu;     // [NK][2F]: d(gate pre-activation) | d(up pre-activation)
  uint16_t* dxp;     // [NK][H]: per-assignment dx (gate and up parts summed)
  float* partial;
  size_t total;
};

struct MoeSaved {
  uint16_t* gu;      // [NK][2F] bf16: gate pre-activation | up pre-activation
  uint16_t* h;       // [NK][F] silu(gate) * up
  uint16_t* su[3];   // s*u planes per projection [2][NK][R]
  size_t total;
};

MoeSaved carve_saved(const moe_shape& sh, void* p) {
  Carve cv(p, 0);
  const size_t NK = (size_t)std::max<int64_t>(sh.n_tokens * sh.top_k, 1);
  MoeSaved m{};
  m.gu = cv.take<uint16_t>(NK * 2 * sh.d_ff);
  m.h = cv.take<uint16_t>(NK * sh.d_ff);
  for (int i = 0; i < 3; ++i) m.su[i] = cv.take<uint16_t>(2 * NK * sh.max_rank);
  m.total = cv.used;
  return m;
}

// routed = false (the MLP layer): one expert, no routing weights; y and dx
// are written straight to token rows, so there is no expert-output buffer.
MoeWs carve_moe(const moe_shape& sh, void* ws, size_t bytes, bool backward, bool routed = true) {
  Carve cv(ws, bytes);
  MoeWs w{};
  const int64_t NK = std::max<int64_t>(sh.n_tokens * sh.top_k, 1);
  const int32_t n_keys = sh.n_experts * (sh.n_adapters + 1);
  const int64_t packs[3] = {sh.gate_pack_elems, sh.up_pack_elems, sh.down_pack_elems};
  w.seg_bytes = segments_ws_bytes(NK, n_keys);
  w.seg = cv.take<char>(w.seg_bytes);
  w.keys = cv.take<int32_t>(NK);
  w.perm = cv.take<int32_t>(NK);
  w.adpos = cv.take<int32_t>(NK);
  w.tokrow = cv.take<int32_t>(NK);
  w.inv = cv.take<int32_t>(NK);
  w.offsets = cv.take<int32_t>((size_t)n_keys + 1);
  w.active = cv.take<uint8_t>((size_t)n_keys);
  w.pre32 = cv.take<int32_t>((size_t)n_keys + 1);
  w.pre128 = cv.take<int32_t>((size_t)n_keys + 1);
  w.prec = cv.take<int32_t>((size_t)n_keys + 1);
  w.gpre = cv.take<int32_t>((size_t)sh.n_experts + 1);
  for (int i = 0; i < 3; ++i) w.desc[i] = cv.take<lora_adapter_desc>((size_t)n_keys);
  w.zero = cv.take<uint16_t>(128);
  if (!backward) {
    if (routed) w.o = cv.take<uint16_t>((size_t)NK * sh.hidden);
  } else {
    w.wpos = cv.take<float>(NK);
    for (int i = 0; i < 3; ++i) w.v[i] = cv.take<uint16_t>((size_t)2 * NK * sh.max_rank);
    w.uw = cv.take<uint16_t>((size_t)2 * NK * sh.max_rank);
    w.dgu = cv.take<uint16_t>((size_t)NK * 2 * sh.d_ff);
    if (routed) w.dxp = cv.take<uint16_t>((size_t)NK * sh.hidden);
    w.partial = cv.take<float>((size_t)grad_partial_floats(NK, n_keys,
                                                          std::max(sh.hidden, sh.d_ff),
                                                          2 * sh.max_rank));
  }
  w.total = cv.used;
  return w;
}

// Composite keys, per-key descriptor tables and the sorted assignment order.
lora_status moe_segments(const moe_shape& sh, const int32_t* experts, const int32_t* ids,
                         const lora_adapter_desc* const desc[3], const MoeWs& w, hipStream_t s) {
  const int64_t NK = sh.n_tokens * sh.top_k;
  const int n_keys = sh.n_experts * (sh.n_adapters + 1);
  TRY(launch_moe_keys(experts, ids, NK, sh.top_k, sh.n_experts, sh.n_adapters, w.keys,
                      (int32_t*)w.seg, s));
  lora_adapter_desc* const dst[3] = {w.desc[0], w.desc[1], w.desc[2]};
  TRY(launch_moe_desc(desc, dst, sh.n_experts, sh.n_adapters, s));
  SegExtras ex{};
  ex.tab[0] = SegDescs{w.desc[0], sh.hidden, sh.d_ff, sh.gate_pack_elems, sh.gate_pack_elems};
  ex.tab[1] = SegDescs{w.desc[1], sh.hidden, sh.d_ff, sh.up_pack_elems, sh.up_pack_elems};
  ex.tab[2] = SegDescs{w.desc[2], sh.d_ff, sh.hidden, sh.down_pack_elems, sh.down_pack_elems};
  ex.n_tabs = 3;
  ex.max_rank = sh.max_rank;
  ex.active = w.active;
  ex.tm[0] = kTmShrink;
  ex.pre[0] = w.pre32;
  ex.tm[1] = kTmShrinkTall;
  ex.pre[1] = w.pre128;
  ex.tm[2] = kGradChunk;
  ex.pre[2] = w.prec;
  ex.adpos = w.adpos;
  ex.row_div = sh.top_k;
  ex.tokrow = w.tokrow;
  ex.inv = w.inv;
  ex.group = sh.n_adapters + 1;
  ex.n_groups = sh.n_experts;
  ex.gpre = w.gpre;
  return run_segments(w.keys, NK, n_keys, LORA_IDS_INTERLEAVED, w.perm, w.offsets, &ex, w.seg,
                      w.seg_bytes, s);
}

// Second weight set of a fused pair of expert projections (gate and up):
// split = 2: K = 2 k_in, the second half of each A row against W2 (backward
// dX, both expands added); split = 3: each tile holds n_out-columns halves of
// gate and up (W2, LoRA set 2), C gets [gate | up] rows and hout = silu(gate) *
// up (forward); split = 4: the product is dh (C nullable) and the epilogue
// turns it into [dgate | dup] rows (dgu) from the saved [gate | up] rows (gu).
struct MoePair {
  int split = 0;
  const uint16_t* W2 = nullptr;
  const uint16_t* planes2 = nullptr;
  const uint16_t* lmat2 = nullptr;
  const lora_adapter_desc* desc2 = nullptr;
  uint16_t* hout = nullptr;
  const uint16_t* gu = nullptr;
  uint16_t* dgu = nullptr;
};

// One grouped expert projection over the sorted assignments: rows gathered
// through a_rows (nullable), base weights per expert, the LoRA expand fused.
lora_status moe_project(const moe_shape& sh, const MoeWs& w, const uint16_t* A,
                        const int32_t* a_rows, int64_t a_rows_bound, const uint16_t* W,
                        int64_t n_out, int64_t k_in, const uint16_t* planes,
                        const uint16_t* lmat, int use_b_off, const lora_adapter_desc* desc,
                        const float* rowscale, uint16_t* C, hipStream_t s,
                        const MoePair& pair = MoePair{}, const int32_t* c_rows = nullptr) {
  const int64_t NK = sh.n_tokens * sh.top_k;
  GemmRows f;
  f.c_rows = c_rows;        // output rows (the LoRA vectors stay in position order)
  f.vec_by_pos = c_rows != nullptr;
  f.B2 = pair.W2;
  f.vec2 = pair.planes2;
  f.lmat2 = pair.lmat2;
  f.desc2 = pair.desc2;
  f.k_split = pair.split == 2 ? (int)k_in : 0;
  f.glu = pair.split == 3 ? 1 : pair.split == 4 ? 2 : 0;
  f.c_off2 = n_out;
  f.hout = pair.hout;
  f.ld_h = n_out;
  f.gu = pair.gu;
  f.ld_gu = 2 * n_out;
  f.dgu = pair.dgu;
  f.ld_dgu = 2 * n_out;
  const int64_t K = pair.split == 2 ? 2 * k_in : k_in;      // columns of A read
  const int64_t lda = a_rows ? k_in : K;                      // gathered rows: x itself
  const int64_t ldc = pair.split == 3 ? 2 * n_out : n_out;
  f.a_rows = a_rows;
  f.a_rows_bound = a_rows_bound;
  f.rowscale = rowscale;
  f.g_tile = w.gpre;
  f.g_off = w.offsets;
  f.g_stride = sh.n_adapters + 1;
  f.n_groups = sh.n_experts;
  f.ldb_group = n_out * k_in;
  f.tiles_m_bound = (int)(cdiv(NK, 256) + sh.n_experts);
  f.vec = planes;
  f.vec_plane = NK * sh.max_rank;
  f.vec_ld = sh.max_rank;
  f.use_b_off = use_b_off;
  f.lmat_ld = n_out;   // A_e,a is [r][n_out] when the expand runs from A
  f.lmat = lmat;
  f.desc = desc;
  f.adpos = w.adpos;
  f.n_ad = sh.n_experts * (sh.n_adapters + 1);
  timer_begin(LORA_TIMER_BASE_GEMM, s);
  TRY(gemm_nt_rows(A, W, C, (int)NK, (int)n_out, (int)K, lda, k_in, ldc, f, s));
  timer_end(LORA_TIMER_BASE_GEMM, s);
  return LORA_OK;
}

}  // namespace

extern "C" {

lora_status moe_route(int64_t n, int32_t n_experts, int32_t top_k, const float* logits,
                      int32_t* experts, float* weights, void* stream) {
  LORA_ARG_CHECK(n >= 0, "n must be >= 0");
  LORA_ARG_CHECK(n_experts >= 1 && n_experts <= 1024, "n_experts %d outside [1, 1024]", n_experts);
  LORA_ARG_CHECK(top_k >= 1 && top_k <= 16 && top_k <= n_experts,
                 "top_k %d outside [1, min(16, n_experts)]", top_k);
  LORA_ARG_CHECK(n == 0 || (logits && experts && weights), "logits/experts/weights NULL");
  return launch_moe_route(logits, n, n_experts, top_k, experts, weights, S(stream));
}

size_t moe_workspace_bytes(const moe_shape* shape) {
  if (check_moe(shape) != LORA_OK) return 0;
  return std::max(carve_moe(*shape, nullptr, 0, false).total,
                  carve_moe(*shape, nullptr, 0, true).total);
}

size_t moe_saved_bytes(const moe_shape* shape) {
  if (check_moe(shape) != LORA_OK) return 0;
  return carve_saved(*shape, nullptr).total;
}

}  // extern "C"

namespace {

// The SwiGLU expert layer behind moe_* (routed: experts and weights given)
// and mlp_* (one expert, experts and weights null: y and dx go straight to
// token rows, no combine).
lora_status expert_forward(const moe_shape& sh, const uint16_t* x, const int32_t* experts,
                           const float* weights, const int32_t* adapter_ids,
                           const uint16_t* W_gate, const uint16_t* W_up, const uint16_t* W_down,
                           const uint16_t* gate_pack, const uint16_t* up_pack,
                           const uint16_t* down_pack, const lora_adapter_desc* gate_desc,
                           const lora_adapter_desc* up_desc, const lora_adapter_desc* down_desc,
                           uint16_t* y, void* saved, void* ws, size_t ws_bytes, hipStream_t s,
                           const char* name) {
  const bool routed = weights != nullptr;
  LORA_ARG_CHECK(W_gate && W_up && W_down && gate_pack && up_pack && down_pack && gate_desc &&
                     up_desc && down_desc,
                 "%s: weights, packs and descriptor tables must be non-NULL", name);
  LORA_ARG_CHECK(sh.n_tokens == 0 || (x && adapter_ids && y && saved),
                 "%s: x, adapter_ids, y and saved must be non-NULL", name);
  LORA_ARG_CHECK(aligned16(x) && aligned16(y) && aligned16(saved) && aligned16(W_gate) &&
                     aligned16(W_up) && aligned16(W_down) && aligned16(gate_pack) &&
                     aligned16(up_pack) && aligned16(down_pack),
                 "%s: activations, weights, packs and saved must be 16-byte aligned", name);
  MoeWs w = carve_moe(sh, ws, ws_bytes, false, routed);
  if (!ws || w.total > ws_bytes) {
    set_error("%s: workspace %zu bytes < %zu needed", name, ws_bytes, w.total);
    return LORA_E_WORKSPACE;
  }
  if (sh.n_tokens == 0) return LORA_OK;
  const MoeSaved sv = carve_saved(sh, saved);
  const int64_t NK = sh.n_tokens * sh.top_k, H = sh.hidden, F = sh.d_ff;
  const int R = sh.max_rank;
  const int n_keys = sh.n_experts * (sh.n_adapters + 1);
  const lora_adapter_desc* const descs[3] = {gate_desc, up_desc, down_desc};
  TRY(moe_segments(sh, experts, adapter_ids, descs, w, s));
  // gate and up: s*u planes from the gathered token rows (one pass over x when
  // both fit one tile), then one grouped GEMM writing [gate | up] rows and h
  if (R <= 32) {
    TRY(launch_shrink(x, H, (int)H, gate_pack, 0, w.desc[0], w.adpos, w.tokrow, nullptr, nullptr,
                      w.offsets, w.pre32, n_keys, NK, sv.su[0], R, w.zero, s, up_pack, w.desc[1],
                      sv.su[1], w.pre128));
  } else {
    TRY(launch_shrink(x, H, (int)H, gate_pack, 0, w.desc[0], w.adpos, w.tokrow, nullptr, nullptr,
                      w.offsets, w.pre32, n_keys, NK, sv.su[0], R, w.zero, s, nullptr, nullptr,
                      nullptr, w.pre128));
    TRY(launch_shrink(x, H, (int)H, up_pack, 0, w.desc[1], w.adpos, w.tokrow, nullptr, nullptr,
                      w.offsets, w.pre32, n_keys, NK, sv.su[1], R, w.zero, s, nullptr, nullptr,
                      nullptr, w.pre128));
  }
  MoePair gu;
  gu.split = 3;
  gu.W2 = W_up;
  gu.planes2 = sv.su[1];
  gu.lmat2 = up_pack;
  gu.desc2 = w.desc[1];
  gu.hout = sv.h;
  TRY(moe_project(sh, w, x, w.tokrow, sh.n_tokens, W_gate, F, H, sv.su[0], gate_pack, 1,
                  w.desc[0], nullptr, sv.gu, s, gu));
  TRY(launch_shrink(sv.h, F, (int)F, down_pack, 0, w.desc[2], w.adpos, nullptr, nullptr, nullptr,
                    w.offsets, w.pre32, n_keys, NK, sv.su[2], R, w.zero, s, nullptr, nullptr,
                    nullptr, w.pre128));
  if (!routed)   // down straight to the token rows
    return moe_project(sh, w, sv.h, nullptr, NK, W_down, H, F, sv.su[2], down_pack, 1, w.desc[2],
                       nullptr, y, s, MoePair{}, w.tokrow);
  // down, then the weighted combine back to tokens
  TRY(moe_project(sh, w, sv.h, nullptr, NK, W_down, H, F, sv.su[2], down_pack, 1, w.desc[2],
                  nullptr, w.o, s));
  return launch_moe_combine(w.o, weights, w.inv, w.keys, sh.n_tokens, sh.top_k, H, y, s);
}

lora_status expert_backward(const moe_shape& sh, const uint16_t* dy, const uint16_t* x,
                            const int32_t* experts, const float* weights,
                            const int32_t* adapter_ids, const uint16_t* W_gate_t,
                            const uint16_t* W_up_t, const uint16_t* W_down_t,
                            const uint16_t* gate_pack, const uint16_t* up_pack,
                            const uint16_t* down_pack, const lora_adapter_desc* gate_desc,
                            const lora_adapter_desc* up_desc, const lora_adapter_desc* down_desc,
                            const void* saved, uint16_t* dx, float* dgate_pack, float* dup_pack,
                            float* ddown_pack, int accumulate, uint16_t* trace, void* ws,
                            size_t ws_bytes, hipStream_t s, const char* name) {
  const bool routed = weights != nullptr;
  LORA_ARG_CHECK(W_gate_t && W_up_t && W_down_t && gate_pack && up_pack && down_pack &&
                     gate_desc && up_desc && down_desc && dgate_pack && dup_pack && ddown_pack,
                 "%s: weights, packs, descriptor tables and gradient packs must be non-NULL", name);
  LORA_ARG_CHECK(sh.n_tokens == 0 || (dy && x && adapter_ids && saved && dx),
                 "%s: dy, x, adapter_ids, saved and dx must be non-NULL", name);
  LORA_ARG_CHECK(aligned16(dy) && aligned16(x) && aligned16(dx) && aligned16(saved) &&
                     aligned16(W_gate_t) && aligned16(W_up_t) && aligned16(W_down_t) &&
                     aligned16(gate_pack) && aligned16(up_pack) && aligned16(down_pack) &&
                     aligned16(dgate_pack) && aligned16(dup_pack) && aligned16(ddown_pack),
                 "%s: activations, weights, packs and saved must be 16-byte aligned", name);
  MoeWs w = carve_moe(sh, ws, ws_bytes, true, routed);
  if (!ws || w.total > ws_bytes) {
    set_error("%s: workspace %zu bytes < %zu needed", name, ws_bytes, w.total);
    return LORA_E_WORKSPACE;
  }
  if (trace) {   // the caller keeps dh and [dgate | dup]
    LORA_ARG_CHECK(aligned16(trace), "%s: trace must be 16-byte aligned", name);
    w.dh = trace;
    w.dgu = trace + sh.n_tokens * sh.top_k * sh.d_ff;
  }
  const MoeSaved sv = carve_saved(sh, const_cast<void*>(saved));
  const int64_t NK = sh.n_tokens * sh.top_k, H = sh.hidden, F = sh.d_ff;
  const int R = sh.max_rank;
  const int n_keys = sh.n_experts * (sh.n_adapters + 1);
  const lora_adapter_desc* const descs[3] = {gate_desc, up_desc, down_desc};
  TRY(moe_segments(sh, experts, adapter_ids, descs, w, s));
  const uint16_t* packs[3] = {gate_pack, up_pack, down_pack};
  float* grads[3] = {dgate_pack, dup_pack, ddown_pack};
  // routed: do_j = w_j dy_t, so v = s w B^T dy_t and u_down enters dB as w s u
  const uint16_t* u_down = routed ? w.uw : sv.su[2];
  if (NK > 0) {
    if (routed) TRY(launch_moe_gather_w(weights, w.perm, NK, w.wpos, s));
    TRY(launch_shrink(dy, H, (int)H, down_pack, 1, w.desc[2], w.adpos, w.tokrow, nullptr,
                      routed ? w.wpos : nullptr, w.offsets, w.pre32, n_keys, NK, w.v[2], R,
                      w.zero, s, nullptr, nullptr, nullptr, w.pre128));
    // dh = w (dy_t W_down) + A^T v, turned into [dgate | dup] in the epilogue
    MoePair dg;
    dg.split = 4;
    dg.gu = sv.gu;
    dg.dgu = w.dgu;
    TRY(moe_project(sh, w, dy, w.tokrow, sh.n_tokens, W_down_t, F, H, w.v[2], down_pack, 0,
                    w.desc[2], routed ? w.wpos : nullptr, w.dh, s, dg));
    if (routed) TRY(launch_planes_scale(sv.su[2], w.wpos, NK, R, w.uw, s));
  }
  // dB_down = sum do_t (s u)^T; dA_down = sum (s v) h^T
  TRY(launch_grad(0, u_down, R, w.zero, dy, H, (int)H, w.desc[2], w.active, w.tokrow, 1,
                  w.offsets, w.prec, n_keys, NK, grads[2], w.partial, accumulate, s));
  TRY(launch_grad(1, w.v[2], R, w.zero, sv.h, F, (int)F, w.desc[2], w.active, nullptr, 1,
                  w.offsets, w.prec, n_keys, NK, grads[2], w.partial, accumulate, s));
  if (NK > 0) {
    // gate and up: v = s B^T d per projection; dx_j = [dg | du] [W_gate; W_up]
    // (one K-concatenated GEMM) + A_gate^T v_gate + A_up^T v_up
    for (int i = 0; i < 2; ++i)
      TRY(launch_shrink(w.dgu + i * F, 2 * F, (int)F, packs[i], 1, w.desc[i], w.adpos, nullptr,
                        nullptr, nullptr, w.offsets, w.pre32, n_keys, NK, w.v[i], R, w.zero, s,
                        nullptr, nullptr, nullptr, w.pre128));
    MoePair gu;
    gu.split = 2;
    gu.W2 = W_up_t;
    gu.planes2 = w.v[1];
    gu.lmat2 = up_pack;
    gu.desc2 = w.desc[1];
    TRY(moe_project(sh, w, w.dgu, nullptr, NK, W_gate_t, H, F, w.v[0], gate_pack, 0, w.desc[0],
                    nullptr, routed ? w.dxp : dx, s, gu, routed ? nullptr : w.tokrow));
  }
  // dB = sum d (s u)^T; dA = sum (s v) x_t^T (gate and up in one pass over x
  // when both fit one tile)
  for (int i = 0; i < 2; ++i)
    TRY(launch_grad(0, sv.su[i], R, w.zero, w.dgu + i * F, 2 * F, (int)F, w.desc[i], w.active,
                    nullptr, 1, w.offsets, w.prec, n_keys, NK, grads[i], w.partial, accumulate, s));
  if (R <= 32) {
    TRY(launch_grad(1, w.v[0], R, w.zero, x, H, (int)H, w.desc[0], w.active, w.tokrow, 1,
                    w.offsets, w.prec, n_keys, NK, grads[0], w.partial, accumulate, s, w.v[1],
                    w.desc[1], grads[1]));
  } else {
    for (int i = 0; i < 2; ++i)
      TRY(launch_grad(1, w.v[i], R, w.zero, x, H, (int)H, w.desc[i], w.active, w.tokrow, 1,
                      w.offsets, w.prec, n_keys, NK, grads[i], w.partial, accumulate, s));
  }
  if (!routed) return LORA_OK;
  return launch_moe_combine(w.dxp, nullptr, w.inv, w.keys, sh.n_tokens, sh.top_k, H, dx,
                            s);
}

moe_shape mlp_as_moe(const mlp_shape& m) {
  moe_shape sh{};
  sh.n_tokens = m.n_tokens;
  sh.hidden = m.hidden;
  sh.d_ff = m.d_ff;
  sh.gate_pack_elems = m.gate_pack_elems;
  sh.up_pack_elems = m.up_pack_elems;
  sh.down_pack_elems = m.down_pack_elems;
  sh.n_experts = 1;
  sh.top_k = 1;
  sh.n_adapters = m.n_adapters;
  sh.max_rank = m.max_rank;
  return sh;
}

lora_status check_mlp(const mlp_shape* shape, moe_shape* out) {
  LORA_ARG_CHECK(shape != nullptr, "mlp shape is NULL");
  *out = mlp_as_moe(*shape);
  return check_moe(out);
}

}  // namespace

extern "C" {

lora_status moe_forward(const moe_shape* shape, const uint16_t* x, const int32_t* experts,
                        const float* weights, const int32_t* adapter_ids, const uint16_t* W_gate,
                        const uint16_t* W_up, const uint16_t* W_down, const uint16_t* gate_pack,
                        const uint16_t* up_pack, const uint16_t* down_pack,
                        const lora_adapter_desc* gate_desc, const lora_adapter_desc* up_desc,
                        const lora_adapter_desc* down_desc, uint16_t* y, void* saved, void* ws,
                        size_t ws_bytes, void* stream) {
  TRY(check_moe(shape));
  LORA_ARG_CHECK(shape->n_tokens == 0 || (experts && weights),
                 "moe_forward: experts and weights must be non-NULL");
  return expert_forward(*shape, x, experts, weights, adapter_ids, W_gate, W_up, W_down, gate_pack,
                        up_pack, down_pack, gate_desc, up_desc, down_desc, y, saved, ws, ws_bytes,
                        S(stream), "moe_forward");
}

lora_status moe_backward(const moe_shape* shape, const uint16_t* dy, const uint16_t* x,
                         const int32_t* experts, const float* weights, const int32_t* adapter_ids,
                         const uint16_t* W_gate_t, const uint16_t* W_up_t,
                         const uint16_t* W_down_t, const uint16_t* gate_pack,
                         const uint16_t* up_pack, const uint16_t* down_pack,
                         const lora_adapter_desc* gate_desc, const lora_adapter_desc* up_desc,
                         const lora_adapter_desc* down_desc, const void* saved, uint16_t* dx,
                         float* dgate_pack, float* dup_pack, float* ddown_pack, int accumulate,
                         uint16_t* trace, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_moe(shape));
  LORA_ARG_CHECK(shape->n_tokens == 0 || (experts && weights),
                 "moe_backward: experts and weights must be non-NULL");
  return expert_backward(*shape, dy, x, experts, weights, adapter_ids, W_gate_t, W_up_t, W_down_t,
                         gate_pack, up_pack, down_pack, gate_desc, up_desc, down_desc, saved, dx,
                         dgate_pack, dup_pack, ddown_pack, accumulate, trace, ws, ws_bytes,
                         S(stream), "moe_backward");
}

size_t mlp_workspace_bytes(const mlp_shape* shape) {
  moe_shape sh;
  if (check_mlp(shape, &sh) != LORA_OK) return 0;
  return std::max(carve_moe(sh, nullptr, 0, false, false).total,
                  carve_moe(sh, nullptr, 0, true, false).total);
}

size_t mlp_saved_bytes(const mlp_shape* shape) {
  moe_shape sh;
  if (check_mlp(shape, &sh) != LORA_OK) return 0;
  return carve_saved(sh, nullptr).total;
}

lora_status mlp_forward(const mlp_shape* shape, const uint16_t* x, const int32_t* adapter_ids,
                        const uint16_t* W_gate, const uint16_t* W_up, const uint16_t* W_down,
                        const uint16_t* gate_pack, const uint16_t* up_pack,
                        const uint16_t* down_pack, const lora_adapter_desc* gate_desc,
                        const lora_adapter_desc* up_desc, const lora_adapter_desc* down_desc,
                        uint16_t* y, void* saved, void* ws, size_t ws_bytes, void* stream) {
  moe_shape sh;
  TRY(check_mlp(shape, &sh));
  return expert_forward(sh, x, nullptr, nullptr, adapter_ids, W_gate, W_up, W_down, gate_pack,
                        up_pack, down_pack, gate_desc, up_desc, down_desc, y, saved, ws, ws_bytes,
                        S(stream), "mlp_forward");
}

lora_status mlp_backward(const mlp_shape* shape, const uint16_t* dy, const uint16_t* x,
                         const int32_t* adapter_ids, const uint16_t* W_gate_t,
                         const uint16_t* W_up_t, const uint16_t* W_down_t,
                         const uint16_t* gate_pack, const uint16_t* up_pack,
                         const uint16_t* down_pack, const lora_adapter_desc* gate_desc,
                         const lora_adapter_desc* up_desc, const lora_adapter_desc* down_desc,
                         const void* saved, uint16_t* dx, float* dgate_pack, float* dup_pack,
                         float* ddown_pack, int accumulate, uint16_t* trace, void* ws,
                         size_t ws_bytes, void* stream) {
  moe_shape sh;
  TRY(check_mlp(shape, &sh));
  return expert_backward(sh, dy, x, nullptr, nullptr, adapter_ids, W_gate_t, W_up_t, W_down_t,
                         gate_pack, up_pack, down_pack, gate_desc, up_desc, down_desc, saved, dx,
                         dgate_pack, dup_pack, ddown_pack, accumulate, trace, ws, ws_bytes,
                         S(stream), "mlp_backward");
}

lora_status bf16_add(int64_t n, const uint16_t* a, const uint16_t* b, uint16_t* out,
                     void* stream) {
  LORA_ARG_CHECK(n >= 0 && (n == 0 || (a && b && out)), "bad bf16_add arguments");
  LORA_ARG_CHECK(n == 0 || (aligned16(a) && aligned16(b) && aligned16(out)),
                 "bf16_add buffers must be 16-byte aligned");
  return launch_add_bf16(n, a, b, out, S(stream));
}

// ------------------------------------------------------------------ timing
void lora_timing_enable(int on) { g_tim.on = on != 0; }

void lora_timing_reset(void) {
  for (int i = 0; i < LORA_TIMER_COUNT; ++i) g_tim.used[i] = 0;
}

lora_status lora_timing_read(int32_t timer, double* total_ms, int64_t* launches) {
  LORA_ARG_CHECK(timer >= 0 && timer < LORA_TIMER_COUNT, "unknown timer %d", timer);
  LORA_ARG_CHECK(total_ms && launches, "NULL output pointer");
  double tot = 0.0;
  const size_t u = g_tim.used[timer];
  for (size_t i = 0; i < u; ++i) {
    auto& pr = g_tim.pairs[timer][i];
    TRY(hip_check(hipEventSynchronize(pr.second), "hipEventSynchronize"));
    float ms = 0.f;
    TRY(hip_check(hipEventElapsedTime(&ms, pr.first, pr.second), "hipEventElapsedTime"));
    tot += ms;
  }
  *total_ms = tot;
  *launches = (int64_t)u;
  return LORA_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ forward without allocation
// lora_forward_noalloc runs lora_forward's kernels on a fixed device array of
// this file instead of a caller workspace.  Each GPU holds its own copy of the
// array (kScratchBytes) from the library's load until the process ends; its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept in g_scratch below -- the array's name in host code
// is only a host-side stand-in and is never handed to a kernel.
namespace {
constexpr size_t kScratchBytes = (size_t)2 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
lora_status scratch_of_current_device(void** out) {
  int dev = -1;
  TRY(hip_check(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("lora_forward_noalloc: device %d outside the %d the scratch table holds", dev,
              kMaxDevices);
    return LORA_E_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    TRY(hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (p == nullptr) {
      set_error("lora_forward_noalloc: no device address for the scratch array");
      return LORA_E_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return LORA_OK;
}
}  // namespace

extern "C" {

size_t lora_forward_noalloc_scratch_bytes(void) { return kScratchBytes; }

lora_status lora_forward_noalloc(const lora_shape* shape, const uint16_t* x, const uint16_t* W,
                                 const uint16_t* A_pack, const uint16_t* B_pack,
                                 const lora_adapter_desc* desc, const int32_t* adapter_ids,
                                 uint16_t* y, uint16_t* u_saved, int32_t* status, void* stream) {
  TRY(forward_checks(shape, x, W, A_pack, B_pack, desc, adapter_ids, y, u_saved));
  const LayerWs need = carve_layer(*shape, nullptr, 0, true);
  if (need.total > kScratchBytes) {
    set_error("lora_forward_noalloc: this shape needs %zu bytes of scratch; the fixed array "
              "holds %zu (e.g. up to 65536 tokens with 1024 adapters)", need.total, kScratchBytes);
    return LORA_E_UNSUPPORTED;
  }
  void* ptr = nullptr;
  TRY(scratch_of_current_device(&ptr));
  const LayerWs w = carve_layer(*shape, ptr, kScratchBytes, true);
  hipStream_t s = S(stream);
  // the status word is the one part of the scratch read before this call writes
  // it: clear it (a fill kernel, so the call can be captured in a graph)
  TRY(launch_fill_i32((int32_t*)ptr, 1, 0, s));
  TRY(forward_core(*shape, x, W, A_pack, B_pack, desc, adapter_ids, y, u_saved, w, s));
  if (status) TRY(launch_or_status((const int32_t*)ptr, status, s));
  return LORA_OK;
}

}  // extern "C"
