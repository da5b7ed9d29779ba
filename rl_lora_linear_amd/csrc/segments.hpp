// Internal interface of the segment builder shared by the layer entry points.
#pragma once
#include "common.hpp"

namespace lora {
constexpr int SEG_CHUNK = 256;  // tokens per histogram/scatter block
}

namespace lora_host {

// A descriptor table the segment builder validates (and its pack bounds).
struct SegDescs {
  const lora_adapter_desc* desc;
  int64_t d_in, d_out, a_elems, b_elems;
};

// Optional extras computed alongside the segment offsets for the LoRA
// kernels: descriptor validation (-> active[]; a key is active when its entry
// is valid in every table; rank 0 marks "no adapter" and is inactive without
// a flag), per-key prefix sums of the number of TM-row tiles and TC-row chunks
// (inactive keys get none), the key of every sorted position, and for
// routed assignments (row_div > 0) the source row item/row_div of every
// position, the inverse permutation, and 256-row tile prefixes over groups of
// `group` consecutive keys.
struct SegExtras {
  SegDescs tab[3];
  int32_t n_tabs;      // 0: every key is active
  int32_t max_rank;
  uint8_t* active;     // out [n_keys]
  int32_t tm[3];       // rows per tile/chunk for up to three tilings
  int32_t* pre[3];     // out [n_keys + 1] each: exclusive prefix of ceil(count / tm)
  int32_t* adpos;      // out [n] (nullable): key of each sorted position, -1 for
                       // invalid ids and inactive keys
  int32_t row_div;     // > 0: routed assignments (item j belongs to row j / row_div)
  int32_t* tokrow;     // out [n]: perm[p] / row_div
  int32_t* inv;        // out [n]: position of item j
  int32_t group;       // keys per group (expert)
  int32_t n_groups;
  int32_t* gpre;       // out [n_groups + 1]: prefix of ceil(group rows / 256)
};

size_t segments_ws_bytes(int64_t n, int32_t n_keys);
// `ws` begins with the status word; the rest is scratch for the sort.
lora_status run_segments(const int32_t* ids, int64_t n, int32_t n_keys, int32_t order,
                         int32_t* perm, int32_t* offsets, SegExtras* ex, void* ws,
                         size_t ws_bytes, hipStream_t s);

}  // namespace lora_host
