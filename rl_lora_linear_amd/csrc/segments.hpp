// Internal interface of the segment builder shared by the layer entry points.
#pragma once
#include "common.hpp"

namespace lora {
constexpr int SEG_CHUNK = 256;  // tokens per histogram/scatter block
}

namespace lora_host {

// Optional extras computed alongside the segment offsets for the LoRA
// kernels: descriptor validation (-> active[]), and per-adapter prefix sums of
// the number of TM-row tiles and TC-row chunks (inactive adapters get none).
struct SegExtras {
  const lora_adapter_desc* desc;  // device, may be null (then every key is active)
  int64_t d_in, d_out, a_elems, b_elems;
  int32_t max_rank;
  uint8_t* active;     // out [n_keys]
  int32_t tm[3];       // rows per tile/chunk for up to three tilings
  int32_t* pre[3];     // out [n_keys + 1] each: exclusive prefix of ceil(count / tm)
  int32_t* adpos;      // out [n] (nullable): key of each sorted position, -1 for
                       // invalid ids and inactive keys
};

size_t segments_ws_bytes(int64_t n, int32_t n_keys);
// `ws` begins with the status word; the rest is scratch for the sort.
lora_status run_segments(const int32_t* ids, int64_t n, int32_t n_keys, int32_t order,
                         int32_t* perm, int32_t* offsets, SegExtras* ex, void* ws,
                         size_t ws_bytes, hipStream_t s);

}  // namespace lora_host
