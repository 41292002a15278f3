// Block-table cell, shared by the block-table kernel and the launch that
// builds the table and the split plan together.
#pragma once

#include "common.h"

namespace mla {

// Cell (b, p) of the block table: the page that holds token 64p of request
// b, or pad_value past the request's pages (and for a req_to_token read that
// would fall outside the map).
__device__ __forceinline__ void block_table_cell(
    int b, int p, const int32_t* __restrict__ req_to_token, int32_t r2t_rows,
    int64_t r2t_row_stride, const int32_t* __restrict__ req_pool_indices,
    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ block_table,
    int32_t bt_row_stride, int32_t pad_value) {
  const int32_t L = seq_lens[b];
  const int32_t npages = L > 0 ? (int32_t)(((int64_t)L + kPage - 1) / kPage) : 0;
  int32_t v = pad_value;
  if (p < npages) {
    const int32_t row = req_pool_indices[b];
    const int64_t col = (int64_t)p * kPage;
    if (row >= 0 && row < r2t_rows && col < r2t_row_stride) {
      const int32_t slot = req_to_token[(int64_t)row * r2t_row_stride + col];
      v = slot >> 6;  // floor(slot / 64), also for negative slots
    }
  }
  block_table[(int64_t)b * bt_row_stride + p] = v;
}

// Argument checks of mla_build_block_table (also run by
// mla_build_table_and_plan); `who` prefixes the error text.
mla_status check_block_table_args(const char* who, const int32_t* req_to_token, int32_t r2t_rows,
                                  int64_t r2t_row_stride, const int32_t* req_pool_indices,
                                  const int32_t* seq_lens, int32_t bs, int32_t page_size,
                                  const int32_t* block_table, int32_t bt_row_stride,
                                  int32_t max_seq_len_hint);

// Argument checks of mla_plan_splits (also run by mla_build_table_and_plan).
mla_status check_plan_args(const char* who, const int32_t* seq_lens, int32_t bs,
                           int32_t rows_per_req, int32_t num_parts, int32_t kv_dtype,
                           const int32_t* tile_plan, const int32_t* split_indptr);

}  // namespace mla
