// Launch of the decode kernel (decode_tile.hip); the argument checks are
// mla_decode's.
#pragma once

#include "common.h"

namespace mla {

struct TileParams {
  int64_t num_pages;
  int32_t partial_slots;  // capacity of partial_o / partial_lse
  int32_t bt_stride;
  int32_t bs;
  int32_t q_len;
  int32_t heads;
  int32_t rows;           // R = q_len * heads
  int32_t causal;
  float scale_log2;       // softmax_scale * log2(e)
};

mla_status launch_tile_decode(const void* q, const void* kv_cache, const int32_t* block_table,
                              const int32_t* seq_lens, const int32_t* tile_plan,
                              int32_t num_parts, const int32_t* split_indptr, void* partial_o,
                              float* partial_lse, void* out, float* lse, const TileParams& p,
                              hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop);

}  // namespace mla
