// Stable counting sort of per-token keys into segments (tinker-ticks, "How
// the SGMV kernel works": one flattened token matrix, a segment index per row).
//
// Four small launches, all deterministic (integer counts only):
//   seg_hist     one block per chunk of 256 tokens: LDS histogram of the
//                chunk's keys (key n_keys collects invalid ids) -> hist[key][chunk];
//                range check and, for sorted input, the monotonicity check.
//   seg_keyscan  one wave per key: exclusive prefix over its chunks (in place)
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

// One wave per key: exclusive prefix of the key's chunk counts (in place, 64
// chunks per pass so the row is read and written coalesced) and its total.
// With descriptor tables, also decide whether key k is usable: in every table,
// rank 8..64, a multiple of 8 and <= max_rank; offsets non-negative, 8-element
// aligned and inside the packs.  A rank of 0 marks "no adapter" (inactive, no
// flag); other unusable entries set LORA_FLAG_BAD_DESC.  Inactive keys are
// treated as having no tokens by the LoRA kernels.
struct SegTabs {
  lora_host::SegDescs tab[3];
  int32_t n_tabs;
};

constexpr int KEYSCAN_WAVES = 4;

__global__ __launch_bounds__(KEYSCAN_WAVES * kWave) void seg_keyscan_kernel(
    int32_t* __restrict__ hist, int n_keys, int n_chunks, int32_t* __restrict__ totals,
    SegTabs tabs, int max_rank, uint8_t* __restrict__ active, int32_t* status) {
  const int lane = threadIdx.x & (kWave - 1);
  const int k = blockIdx.x * KEYSCAN_WAVES + (int)(threadIdx.x / kWave);  // wave-uniform
  if (k > n_keys) return;
  if (tabs.n_tabs > 0 && k < n_keys && lane == 0) {
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
  for (int c0 = 0; c0 < n_chunks; c0 += kWave) {
    const int c = c0 + lane;
    const int32_t v = c < n_chunks ? row[c] : 0;
    int32_t x = v;  // inclusive scan across the wave
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int32_t y = __shfl_up(x, o, kWave);
      if (lane >= o) x += y;
    }
    if (c < n_chunks) row[c] = run + x - v;
    run += __shfl(x, kWave - 1, kWave);
  }
  if (lane == 0) totals[k] = run;
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

// The whole builder in one block of 1024 threads for small batches (one
// launch instead of four).  Chunks are the 64 tokens of one wave: a wave
// counts each distinct key of its chunk with one ballot (no same-address LDS
// atomics, which serialise badly when a chunk's keys are all equal), the
// per-key prefix over chunks and the key scan follow, and a token's place is
// offsets[key] + its chunk's prefix + the lanes below it holding the same key.
constexpr int SEG_SMALL_N = 16384;
constexpr int SEG_SMALL_KEYS = 1024;
constexpr int SEG_SMALL_HIST = 12288;   // chunks * (n_keys + 1) bound (48 KB of LDS)

__device__ __forceinline__ void block_scan4_1024(int32_t (&acc)[4], int32_t (*s_v)[1024]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) s_v[q][tid] = acc[q];
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int32_t x[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = tid >= o ? s_v[q][tid - o] : 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) s_v[q][tid] += x[q];
    __syncthreads();
  }
}

// Lanes of this wave (among `active`) holding the same key as this lane.
__device__ __forceinline__ uint64_t same_key_lanes(int key, uint64_t active, int nbits) {
  // one key in the whole wave (sorted ids): one ballot
  const int k0 = __builtin_amdgcn_readfirstlane(key);
  if (__ballot(key == k0) == ~0ull) return active;
  // else the lanes whose key agrees with this lane's in every one of its nbits
  // bits: one ballot per bit, no loop over the distinct keys of the wave
  uint64_t m = active;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t on = __ballot(bit);
    m &= bit ? on : ~on;
  }
  return m;
}

__global__ __launch_bounds__(1024) void seg_small_kernel(
    const int32_t* __restrict__ ids, int n, int n_keys, int sorted, SegTabs tabs, int max_rank,
    uint8_t* __restrict__ active, Tilings tl, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ adpos, int row_div,
    int32_t* __restrict__ tokrow, int32_t* __restrict__ inv, int32_t* status) {
  __shared__ int32_t s_v[4][1024];
  __shared__ int32_t s_off[SEG_SMALL_KEYS + 1];
  __shared__ uint8_t s_act[SEG_SMALL_KEYS + 1];
  __shared__ int32_t s_ids[SEG_SMALL_N];
  extern __shared__ int32_t s_hist[];   // [chunks of 64][n_keys + 1]
  const int tid = threadIdx.x, lane = tid & 63;
  const int K1 = n_keys + 1;
  const int chunks = (n + 63) / 64;
  const int rounds = (n + 1023) / 1024;
  const int nbits = 32 - __clz(n_keys);   // keys 0..n_keys (n_keys: ids out of range)
  {  // all id loads in flight at once, then into LDS
    int32_t v[SEG_SMALL_N / 1024];
#pragma unroll
    for (int r = 0; r < SEG_SMALL_N / 1024; ++r) {
      const int t = r * 1024 + tid;
      v[r] = t < n ? ids[t] : 0;
    }
    // per key: descriptor validation, its loads issued behind the id loads so
    // that both latencies overlap
    for (int k = tid; k <= n_keys; k += 1024) {
      lora_adapter_desc d[3];
#pragma unroll
      for (int i = 0; i < 3; ++i)
        if (k < n_keys && i < tabs.n_tabs) d[i] = tabs.tab[i].desc[k];
      bool on = true;
      if (k < n_keys && tabs.n_tabs > 0) {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          if (i >= tabs.n_tabs) break;
          const lora_host::SegDescs& tb = tabs.tab[i];
          const int64_t rk = d[i].rank;
          if (rk == 0) {
            on = false;
            continue;
          }
          const bool ok = rk >= 8 && rk <= 64 && (rk % 8) == 0 && rk <= max_rank &&
                          d[i].a_off >= 0 && d[i].b_off >= 0 && (d[i].a_off % 8) == 0 &&
                          (d[i].b_off % 8) == 0 && d[i].a_off + rk * tb.d_in <= tb.a_elems &&
                          d[i].b_off + tb.d_out * rk <= tb.b_elems;
          if (!ok) set_flag(status, LORA_FLAG_BAD_DESC);
          on = on && ok;
        }
        active[k] = on ? 1 : 0;
      }
      s_act[k] = on ? 1 : 0;
    }
#pragma unroll
    for (int r = 0; r < SEG_SMALL_N / 1024; ++r)
      if (r * 1024 + tid < n) s_ids[r * 1024 + tid] = v[r];
  }
  __syncthreads();
  // Sorted ids that are all in range and non-decreasing (the promise kept):
  // the stable order is the identity, and each key's count is the distance
  // between the first positions of consecutive keys.  No histogram, no
  // scatter; the results are those of the general path below.
  bool fast = false;
  if (sorted) {
    int bad = 0;
    for (int r = 0; r < rounds; ++r) {
      const int t = r * 1024 + tid;
      if (t < n) {
        const int32_t id = s_ids[t];
        bad |= (id < 0 || id >= n_keys || (t + 1 < n && s_ids[t + 1] < id)) ? 1 : 0;
      }
    }
    fast = __syncthreads_or(bad) == 0;
  }
  if (fast) {
    // s_off[k] = first position whose id >= k (k = 0..n_keys): each key is
    // written by the one position where the ids step over it
    for (int r = 0; r < rounds; ++r) {
      const int t = r * 1024 + tid;
      if (t < n) {
        const int32_t id = s_ids[t], prev = t ? s_ids[t - 1] : -1;
        for (int k = prev + 1; k <= id; ++k) s_off[k] = t;
        if (t == n - 1)
          for (int k = id + 1; k <= n_keys; ++k) s_off[k] = n;
      }
    }
    __syncthreads();
    const int cnt = tid < n_keys ? s_off[tid + 1] - s_off[tid] : 0;
    __syncthreads();
    if (tid < n_keys) s_off[tid] = cnt;   // counts, as the general path leaves them
    __syncthreads();
  } else {
  for (int i = tid; i < chunks * K1; i += 1024) s_hist[i] = 0;
  __syncthreads();
  for (int r = 0; r < rounds; ++r) {
    const int t = r * 1024 + tid;
    const bool in = t < n;
    int key = n_keys;
    if (in) {
      const int32_t id = s_ids[t];
      key = (id >= 0 && id < n_keys) ? id : n_keys;
      if (key == n_keys) set_flag(status, LORA_FLAG_ID_RANGE);
      if (sorted && t + 1 < n && s_ids[t + 1] < id) set_flag(status, LORA_FLAG_UNSORTED);
    }
    const uint64_t act = __ballot(in);
    const uint64_t same = same_key_lanes(key, act, nbits);
    // the lowest lane of each key group writes the chunk's count
    if (in && (same & ((1ull << lane) - 1)) == 0) s_hist[(t >> 6) * K1 + key] = __popcll(same);
  }
  __syncthreads();
  // per key, one wave: prefix over chunks (in place, 64 chunks per step with a
  // wave scan) and the total (kept in s_off)
  for (int k = tid >> 6; k <= n_keys; k += 16) {
    int32_t base = 0;
    for (int c0 = 0; c0 < chunks; c0 += 64) {
      const int c = c0 + lane;
      const int32_t v = c < chunks ? s_hist[c * K1 + k] : 0;
      int32_t x = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      if (c < chunks) s_hist[c * K1 + k] = base + x - v;
      base += __shfl(x, 63);
    }
    if (lane == 0) s_off[k] = base;
  }
  __syncthreads();
  }
  // exclusive scan over keys: offsets and the tile prefix arrays
  if (n_keys <= 64) {   // one wave, no barriers
    if (tid < 64) {
      const int k = lane;
      const bool kin = k < n_keys;
      const int32_t cnt = kin ? s_off[k] : 0;
      const bool on = kin && s_act[k] != 0;
      int32_t v[4] = {cnt, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 3; ++i)
        if (tl.pre[i]) v[1 + i] = on ? (cnt + tl.tm[i] - 1) / tl.tm[i] : 0;
      int32_t x[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
      for (int o = 1; o < 64; o <<= 1)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int32_t y = __shfl_up(x[q], o);
          if (lane >= o) x[q] += y;
        }
      if (kin) {
        offsets[k] = x[0] - v[0];
        s_off[k] = x[0] - v[0];
#pragma unroll
        for (int i = 0; i < 3; ++i)
          if (tl.pre[i]) tl.pre[i][k] = x[1 + i] - v[1 + i];
      }
      if (lane == 63) {
        offsets[n_keys] = x[0];
        s_off[n_keys] = x[0];
#pragma unroll
        for (int i = 0; i < 3; ++i)
          if (tl.pre[i]) tl.pre[i][n_keys] = x[1 + i];
      }
    }
    __syncthreads();
  } else {
  const int per = (n_keys + 1023) / 1024;
  const int k0 = min(tid * per, n_keys), k1 = min(k0 + per, n_keys);
  int32_t acc[4] = {0, 0, 0, 0};
  for (int k = k0; k < k1; ++k) {
    const int32_t cnt = s_off[k];
    const bool on = s_act[k] != 0;
    acc[0] += cnt;
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (tl.pre[i]) acc[1 + i] += on ? (cnt + tl.tm[i] - 1) / tl.tm[i] : 0;
  }
  block_scan4_1024(acc, s_v);
  int32_t run[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) run[q] = tid ? s_v[q][tid - 1] : 0;
  for (int k = k0; k < k1; ++k) {
    const int32_t cnt = s_off[k];
    const bool on = s_act[k] != 0;
    offsets[k] = run[0];
    s_off[k] = run[0];
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
    s_off[n_keys] = s_v[0][1023];
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (tl.pre[i]) tl.pre[i][n_keys] = s_v[1 + i][1023];
  }
  __syncthreads();
  }
  if (fast) {   // the identity order
    for (int r = 0; r < rounds; ++r) {
      const int t = r * 1024 + tid;
      if (t >= n) continue;
      const int32_t id = s_ids[t];
      perm[t] = t;
      if (adpos) adpos[t] = s_act[id] ? id : -1;
      if (row_div > 0) {
        tokrow[t] = t / row_div;
        inv[t] = t;
      }
    }
    return;
  }
  // scatter, stable within each key
  for (int r = 0; r < rounds; ++r) {
    const int t = r * 1024 + tid;
    const bool in = t < n;
    int key = n_keys;
    if (in) {
      const int32_t id = s_ids[t];
      key = (id >= 0 && id < n_keys) ? id : n_keys;
    }
    const uint64_t same = same_key_lanes(key, __ballot(in), nbits);
    if (!in) continue;
    const int pos = s_off[key] + s_hist[(t >> 6) * K1 + key] + __popcll(same & ((1ull << lane) - 1));
    perm[pos] = t;
    if (adpos) adpos[pos] = (key < n_keys && s_act[key]) ? key : -1;
    if (row_div > 0) {
      tokrow[pos] = t / row_div;
      inv[t] = pos;
    }
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
  SegTabs tabs{};
  if (ex) {
    tabs.n_tabs = ex->n_tabs;
    for (int i = 0; i < ex->n_tabs; ++i) tabs.tab[i] = ex->tab[i];
  }
  Tilings tl{};
  for (int i = 0; i < 3; ++i) {
    tl.tm[i] = (ex && ex->pre[i]) ? ex->tm[i] : 1;
    tl.pre[i] = ex ? ex->pre[i] : nullptr;
  }
  const int64_t chunks64 = cdiv(n, 64);
  if (n > 0 && n <= SEG_SMALL_N && n_keys <= SEG_SMALL_KEYS &&
      chunks64 * (n_keys + 1) <= SEG_SMALL_HIST) {
    // one launch
    const size_t hl = (size_t)chunks64 * (n_keys + 1) * sizeof(int32_t);
    // the kernel's dynamic LDS bound, raised once to the largest histogram this
    // path takes (a thread-safe one-time initialisation, then read-only)
    static const hipError_t attr_err = hipFuncSetAttribute(
        (const void*)seg_small_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)(SEG_SMALL_HIST * sizeof(int32_t)));
    TRY_HIP(attr_err);
    hipLaunchKernelGGL(seg_small_kernel, dim3(1), dim3(1024), hl, s, ids, (int)n, n_keys,
                       order == LORA_IDS_SORTED ? 1 : 0, tabs, ex ? ex->max_rank : 0,
                       ex ? ex->active : nullptr, tl, offsets, perm, ex ? ex->adpos : nullptr,
                       ex ? ex->row_div : 0, ex ? ex->tokrow : nullptr, ex ? ex->inv : nullptr,
                       status);
    lora_status st = launch_check("seg_small");
    if (st) return st;
    if (ex && ex->gpre) {
      hipLaunchKernelGGL(seg_group_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, ex->group,
                         ex->n_groups, ex->gpre);
      st = launch_check("seg_group_tiles");
    }
    return st;
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
  hipLaunchKernelGGL(seg_keyscan_kernel, dim3((unsigned)cdiv(n_keys + 1, KEYSCAN_WAVES)),
                     dim3(KEYSCAN_WAVES * kWave), 0, s,
                     hist, n_keys, (int)chunks, totals, tabs, ex ? ex->max_rank : 0,
                     ex ? ex->active : nullptr, status);
  lora_status st = launch_check("seg_keyscan");
  if (st) return st;
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
