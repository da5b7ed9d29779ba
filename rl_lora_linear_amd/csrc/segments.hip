// Stable counting sort of per-token keys into segments (tinker-ticks, "How
// the SGMV kernel works": one flattened token matrix, a segment index per row).
//
// Four small launches, all deterministic (integer counts only):
//   seg_hist     one block per chunk of 256 tokens: LDS histogram of the
//                chunk's keys (key n_keys collects invalid ids) -> hist[key][chunk];
//                range check and, for sorted input, the monotonicity check.
//   seg_keyscan  one thread per key: exclusive prefix over its chunks (in place)
//                and the key total.
//   seg_offsets  one block: exclusive scan of the key totals -> offsets, plus
//                the per-key tile/chunk prefix sums the LoRA kernels index by.
//   seg_scatter  one block per chunk: each token's place = offsets[key] +
//                prefix[key][chunk] + (earlier tokens of the chunk with that
//                key), so the order inside a key is the token order.
#include "common.hpp"
#include "segments.hpp"

namespace lora {

__global__ __launch_bounds__(SEG_CHUNK) void seg_hist_kernel(const int32_t* __restrict__ ids,
                                                             int64_t n, int n_keys, int sorted,
                                                             int32_t* __restrict__ hist,
                                                             int n_chunks, int32_t* status) {
  extern __shared__ int32_t h_s[];  // [n_keys + 1]
  const int c = blockIdx.x;
  for (int k = threadIdx.x; k <= n_keys; k += blockDim.x) h_s[k] = 0;
  __syncthreads();
  const int64_t t = (int64_t)c * SEG_CHUNK + threadIdx.x;
  if (t < n) {
    int32_t id = ids[t];
    int key = (id >= 0 && id < n_keys) ? id : n_keys;
    if (key == n_keys) set_flag(status, LORA_FLAG_ID_RANGE);
    if (sorted && t + 1 < n && ids[t + 1] < id) set_flag(status, LORA_FLAG_UNSORTED);
    atomicAdd(&h_s[key], 1);
  }
  __syncthreads();
  for (int k = threadIdx.x; k <= n_keys; k += blockDim.x) hist[(int64_t)k * n_chunks + c] = h_s[k];
}

__global__ void seg_zero_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t j = i; j < n; j += (int64_t)gridDim.x * blockDim.x) p[j] = 0;
}

// One thread per key: exclusive prefix of the key's chunk counts (in place)
// and its total.  With descriptor tables, also decide whether key k is
// usable: in every table, rank 8..64, a multiple of 8 and <= max_rank;
// offsets non-negative, 8-element aligned and inside the packs.  A rank of 0
// marks "no adapter" (inactive, no flag); other unusable entries set
// LORA_FLAG_BAD_DESC.  Inactive keys are treated as having no tokens by the
// LoRA kernels.
struct SegTabs {
  lora_host::SegDescs tab[3];
  int32_t n_tabs;
};

__global__ void seg_keyscan_kernel(int32_t* __restrict__ hist, int n_keys, int n_chunks,
                                   int32_t* __restrict__ totals, SegTabs tabs, int max_rank,
                                   uint8_t* __restrict__ active, int32_t* status) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k > n_keys) return;
  if (tabs.n_tabs > 0 && k < n_keys) {
    bool on = true;
    for (int i = 0; i < tabs.n_tabs; ++i) {
      const lora_host::SegDescs& t = tabs.tab[i];
      const lora_adapter_desc d = t.desc[k];
      const int64_t r = d.rank;
      if (r == 0) {
        on = false;
        continue;
      }
      const bool ok = r >= 8 && r <= 64 && (r % 8) == 0 && r <= max_rank && d.a_off >= 0 &&
                      d.b_off >= 0 && (d.a_off % 8) == 0 && (d.b_off % 8) == 0 &&
                      d.a_off + r * t.d_in <= t.a_elems && d.b_off + t.d_out * r <= t.b_elems;
      if (!ok) set_flag(status, LORA_FLAG_BAD_DESC);
      on = on && ok;
    }
    active[k] = on ? 1 : 0;
  }
  int32_t* row = hist + (int64_t)k * n_chunks;
  int32_t run = 0;
  for (int c = 0; c < n_chunks; ++c) {
    int32_t v = row[c];
    row[c] = run;
    run += v;
  }
  totals[k] = run;
}

// One block of 1024 threads: exclusive scan of the key totals -> offsets.
// With tilings, also the exclusive prefix sums of ceil(count / tm[i]) per key
// (0 for inactive keys): block b of a LoRA launch finds its adapter by binary
// search in such a prefix array.
struct Tilings {
  int32_t tm[3];
  int32_t* pre[3];
};

__global__ __launch_bounds__(1024) void seg_offsets_kernel(const int32_t* __restrict__ totals,
                                                           int n_keys,
                                                           int32_t* __restrict__ offsets,
                                                           const uint8_t* __restrict__ active,
                                                           Tilings tl) {
  __shared__ int32_t s_v[4][1024];
  const int tid = threadIdx.x;
  const int per = (n_keys + 1024 - 1) / 1024;
  const int k0 = tid * per;
  const int k1 = min(k0 + per, n_keys);
  int32_t acc[4] = {0, 0, 0, 0};
  for (int k = k0; k < k1; ++k) {
    const int32_t cnt = totals[k];
    const bool on = active ? active[k] != 0 : true;
    acc[0] += cnt;
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (tl.pre[i]) acc[1 + i] += on ? (cnt + tl.tm[i] - 1) / tl.tm[i] : 0;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) s_v[q][tid] = acc[q];
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 per-thread sums
  for (int o = 1; o < 1024; o <<= 1) {
    int32_t x[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = tid >= o ? s_v[q][tid - o] : 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) s_v[q][tid] += x[q];
    __syncthreads();
  }
  int32_t run[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) run[q] = tid ? s_v[q][tid - 1] : 0;
  for (int k = k0; k < k1; ++k) {
    const int32_t cnt = totals[k];
    const bool on = active ? active[k] != 0 : true;
    offsets[k] = run[0];
    run[0] += cnt;
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (tl.pre[i]) {
        tl.pre[i][k] = run[1 + i];
        run[1 + i] += on ? (cnt + tl.tm[i] - 1) / tl.tm[i] : 0;
      }
  }
  if (tid == 1023) {
    offsets[n_keys] = s_v[0][1023];
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (tl.pre[i]) tl.pre[i][n_keys] = s_v[1 + i][1023];
  }
}

__global__ __launch_bounds__(SEG_CHUNK) void seg_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t n, int n_keys, const int32_t* __restrict__ hist,
    int n_chunks, const int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    const uint8_t* __restrict__ active, int32_t* __restrict__ adpos, int row_div,
    int32_t* __restrict__ tokrow, int32_t* __restrict__ inv) {
  __shared__ int32_t k_s[SEG_CHUNK];
  const int c = blockIdx.x;
  const int64_t t = (int64_t)c * SEG_CHUNK + threadIdx.x;
  int key = -1;
  if (t < n) {
    int32_t id = ids[t];
    key = (id >= 0 && id < n_keys) ? id : n_keys;
  }
  k_s[threadIdx.x] = key;
  __syncthreads();
  if (t >= n) return;
  int rank = 0;
  for (int j = 0; j < (int)threadIdx.x; ++j) rank += (k_s[j] == key);
  const int32_t base = (key < n_keys ? offsets[key] : offsets[n_keys]) +
                       hist[(int64_t)key * n_chunks + c];
  perm[base + rank] = (int32_t)t;
  if (adpos) adpos[base + rank] = (key < n_keys && (!active || active[key])) ? key : -1;
  if (row_div > 0) {
    tokrow[base + rank] = (int32_t)(t / row_div);
    inv[t] = base + rank;
  }
}

// One block: gpre[g] = sum over groups g' < g of ceil(rows of g' / 256), where
// group g is keys [g*group, (g+1)*group).  n_groups <= 1024.
__global__ __launch_bounds__(1024) void seg_group_tiles_kernel(const int32_t* __restrict__ offsets,
                                                               int group, int n_groups,
                                                               int32_t* __restrict__ gpre) {
  __shared__ int32_t s_v[1024];
  const int g = threadIdx.x;
  int32_t v = 0;
  if (g < n_groups) v = (offsets[(g + 1) * group] - offsets[g * group] + 255) / 256;
  s_v[g] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t x = g >= o ? s_v[g - o] : 0;
    __syncthreads();
    s_v[g] += x;
    __syncthreads();
  }
  if (g < n_groups) gpre[g + 1] = s_v[g];
  if (g == 0) gpre[0] = 0;
}

}  // namespace lora

namespace lora_host {
using namespace lora;

size_t segments_ws_bytes(int64_t n, int32_t n_keys) {
  Carve cv(nullptr, 0);
  cv.take<int32_t>(64);                                        // status word (+ pad)
  const int64_t chunks = cdiv(n > 0 ? n : 1, SEG_CHUNK);
  cv.take<int32_t>((size_t)(n_keys + 1) * chunks);             // hist
  cv.take<int32_t>((size_t)n_keys + 1);                        // totals
  return cv.used;
}

lora_status run_segments(const int32_t* ids, int64_t n, int32_t n_keys, int32_t order,
                         int32_t* perm, int32_t* offsets, SegExtras* ex, void* ws,
                         size_t ws_bytes, hipStream_t s) {
  Carve cv(ws, ws_bytes);
  int32_t* status = cv.take<int32_t>(64);
  const int64_t chunks = cdiv(n > 0 ? n : 1, SEG_CHUNK);
  int32_t* hist = cv.take<int32_t>((size_t)(n_keys + 1) * chunks);
  int32_t* totals = cv.take<int32_t>((size_t)n_keys + 1);
  if (!cv.fits()) {
    set_error("segments: workspace of %zu bytes < %zu needed", ws_bytes, cv.used);
    return LORA_E_WORKSPACE;
  }
  const size_t lds = (size_t)(n_keys + 1) * sizeof(int32_t);
  if (n > 0) {
    hipLaunchKernelGGL(seg_hist_kernel, dim3((unsigned)chunks), dim3(SEG_CHUNK), lds, s, ids, n,
                       n_keys, order == LORA_IDS_SORTED ? 1 : 0, hist, (int)chunks, status);
    lora_status st = launch_check("seg_hist");
    if (st) return st;
  } else {
    // n == 0: a histogram of zeros (every key empty)
    hipLaunchKernelGGL(seg_zero_kernel, dim3((unsigned)cdiv(n_keys + 1, 256)), dim3(256), 0, s,
                       hist, (int64_t)(n_keys + 1) * chunks);
    lora_status st = launch_check("seg_zero");
    if (st) return st;
  }
  SegTabs tabs{};
  if (ex) {
    tabs.n_tabs = ex->n_tabs;
    for (int i = 0; i < ex->n_tabs; ++i) tabs.tab[i] = ex->tab[i];
  }
  hipLaunchKernelGGL(seg_keyscan_kernel, dim3((unsigned)cdiv(n_keys + 1, 256)), dim3(256), 0, s,
                     hist, n_keys, (int)chunks, totals, tabs, ex ? ex->max_rank : 0,
                     ex ? ex->active : nullptr, status);
  lora_status st = launch_check("seg_keyscan");
  if (st) return st;
  Tilings tl{};
  for (int i = 0; i < 3; ++i) {
    tl.tm[i] = (ex && ex->pre[i]) ? ex->tm[i] : 1;
    tl.pre[i] = ex ? ex->pre[i] : nullptr;
  }
  hipLaunchKernelGGL(seg_offsets_kernel, dim3(1), dim3(1024), 0, s, totals, n_keys, offsets,
                     (ex && ex->n_tabs > 0) ? ex->active : nullptr, tl);
  st = launch_check("seg_offsets");
  if (st) return st;
  if (n > 0) {
    hipLaunchKernelGGL(seg_scatter_kernel, dim3((unsigned)chunks), dim3(SEG_CHUNK), 0, s, ids, n,
                       n_keys, hist, (int)chunks, offsets, perm,
                       (ex && ex->n_tabs > 0) ? ex->active : nullptr, ex ? ex->adpos : nullptr,
                       ex ? ex->row_div : 0, ex ? ex->tokrow : nullptr, ex ? ex->inv : nullptr);
    st = launch_check("seg_scatter");
    if (st) return st;
  }
  if (ex && ex->gpre) {
    hipLaunchKernelGGL(seg_group_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, ex->group,
                       ex->n_groups, ex->gpre);
    st = launch_check("seg_group_tiles");
  }
  return st;
}

}  // namespace lora_host
