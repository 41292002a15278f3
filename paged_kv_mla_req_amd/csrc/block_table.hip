// Block table: the page that holds token 64p of each request, then padding.
//
// This is the index kernel the FlashMLA backend launches once per batch step
// in init_forward_metadata (decode and target-verify branches) and again into
// a fixed-width buffer on graph replay.  One thread per (request, page cell);
// a request's row is written in full, so the table is a pure function of the
// inputs.
#include "block_table.h"

namespace mla {

__global__ void __launch_bounds__(256)
build_block_table_kernel(const int32_t* __restrict__ req_to_token, int32_t r2t_rows,
                         int64_t r2t_row_stride, const int32_t* __restrict__ req_pool_indices,
                         const int32_t* __restrict__ seq_lens, int32_t* __restrict__ block_table,
                         int32_t bt_row_stride, int32_t pad_value) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= bt_row_stride) return;
  block_table_cell(blockIdx.y, p, req_to_token, r2t_rows, r2t_row_stride, req_pool_indices,
                   seq_lens, block_table, bt_row_stride, pad_value);
}

mla_status check_block_table_args(const char* who, const int32_t* req_to_token, int32_t r2t_rows,
                                  int64_t r2t_row_stride, const int32_t* req_pool_indices,
                                  const int32_t* seq_lens, int32_t bs, int32_t page_size,
                                  const int32_t* block_table, int32_t bt_row_stride,
                                  int32_t max_seq_len_hint) {
  const std::string w(who);
  if (!req_to_token || !req_pool_indices || !seq_lens || !block_table)
    return fail(MLA_ERR_INVALID_ARGUMENT, w + ": null pointer");
  if (bs <= 0 || r2t_rows <= 0 || r2t_row_stride <= 0 || bt_row_stride <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, w + ": sizes must be positive");
  if (page_size != kPage)
    return fail(MLA_ERR_UNSUPPORTED, w + ": page_size must be 64");
  if (bs > 65535)
    return fail(MLA_ERR_UNSUPPORTED, w + ": bs above 65535");
  if (max_seq_len_hint >= 0) {
    const int64_t need = ((int64_t)max_seq_len_hint + kPage - 1) / kPage;
    if (need > bt_row_stride)
      return fail(MLA_ERR_CAPACITY,
                  w + ": block table narrower than " + std::to_string(need) + " pages");
    if (need > 0 && (need - 1) * kPage >= r2t_row_stride)
      return fail(MLA_ERR_CAPACITY, w + ": req_to_token rows too short");
  }
  return MLA_OK;
}

}  // namespace mla

extern "C" mla_status mla_build_block_table(const int32_t* req_to_token, int32_t r2t_rows,
                                            int64_t r2t_row_stride,
                                            const int32_t* req_pool_indices,
                                            const int32_t* seq_lens, int32_t bs,
                                            int32_t page_size, int32_t* block_table,
                                            int32_t bt_row_stride, int32_t pad_value,
                                            int32_t max_seq_len_hint, hipStream_t stream) {
  using namespace mla;
  const mla_status st = check_block_table_args(
      "mla_build_block_table", req_to_token, r2t_rows, r2t_row_stride, req_pool_indices,
      seq_lens, bs, page_size, block_table, bt_row_stride, max_seq_len_hint);
  if (st != MLA_OK) return st;
  dim3 grid((bt_row_stride + 255) / 256, bs);
  trace("mla_build_block_table: bs %d width %d grid %ux%u stream %p", bs, bt_row_stride, grid.x,
        grid.y, (void*)stream);
  hipLaunchKernelGGL(build_block_table_kernel, grid, dim3(256), 0, stream, req_to_token,
                     r2t_rows, r2t_row_stride, req_pool_indices, seq_lens, block_table,
                     bt_row_stride, pad_value);
#ifdef MLA_DEBUG
  const mla_status launched = check_launch("mla_build_block_table");
  if (launched != MLA_OK) return launched;
  return debug_check_page_aligned("mla_build_block_table", req_to_token, r2t_rows, r2t_row_stride,
                                  req_pool_indices, seq_lens, bs, block_table, bt_row_stride,
                                  stream);
#else
  return check_launch("mla_build_block_table");
#endif
}
