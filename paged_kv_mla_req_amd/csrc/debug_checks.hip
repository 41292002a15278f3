// Checks of the debug build (libmla_decode_debug.so, compiled with
// -DMLA_DEBUG): preconditions that the release build takes on trust, checked
// on the device before or after the real launch.
//
//  * Page-aligned slots.  The block table holds, for page p of a request, the
//    page of the slot of token 64p (the index kernel of the FlashMLA backend
//    page's init_forward_metadata); the kernels then read token j at
//    64 * table[j / 64] + j % 64, which is right only when the request's
//    tokens sit page-aligned in the pool (forward_decode views the cache as
//    [-1, 64, 1, 576] pages).  The check compares every token's
//    req_to_token slot with that address.
//  * Block-table entries.  Every entry a decode reads (page p of request b,
//    p < ceil(L_b / 64)) lies within the table's width and names a page of
//    the pool.  (The release decode masks such pages; a debug build reports
//    them.)
//
// A violation is recorded in a device error word, the smallest
// (request << 32 | token or page) found; the host reads the word back
// (synchronising the stream) and returns MLA_ERR_PRECONDITION naming the
// first violation.  Debug builds only: the read-back is a host sync.
#include <string>

#include "common.h"

namespace mla {
namespace {

constexpr unsigned long long kNone = ~0ull;
static __device__ unsigned long long g_error_word;

__global__ void reset_word(unsigned long long* word) { *word = kNone; }

__device__ __forceinline__ void record(unsigned long long* word, int b, int j) {
  atomicMin(word, ((unsigned long long)(unsigned)b << 32) | (unsigned)j);
}

// grid (kCheckBlocks, bs), 256 threads: tokens j of request blockIdx.y
__global__ void page_aligned_kernel(const int32_t* req_to_token, int32_t r2t_rows,
                                    int64_t r2t_row_stride, const int32_t* req_pool_indices,
                                    const int32_t* seq_lens, const int32_t* block_table,
                                    int32_t bt_row_stride, unsigned long long* word) {
  const int b = blockIdx.y;
  const int L = seq_lens[b];
  const int row = req_pool_indices[b];
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < L; j += gridDim.x * blockDim.x) {
    if (row < 0 || row >= r2t_rows || j >= r2t_row_stride || j / kPage >= bt_row_stride) {
      record(word, b, j);
      continue;
    }
    const int64_t slot = req_to_token[(int64_t)row * r2t_row_stride + j];
    const int64_t want = (int64_t)block_table[(int64_t)b * bt_row_stride + j / kPage] * kPage +
                         j % kPage;
    if (slot < 0 || slot != want) record(word, b, j);
  }
}

// grid (kCheckBlocks, bs): pages p of request blockIdx.y
__global__ void table_entries_kernel(const int32_t* block_table, int32_t bt_row_stride,
                                     const int32_t* seq_lens, int64_t num_pages,
                                     unsigned long long* word) {
  const int b = blockIdx.y;
  const int L = seq_lens[b];
  const int pages = L > 0 ? (L + kPage - 1) / kPage : 0;
  for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < pages; p += gridDim.x * blockDim.x) {
    if (p >= bt_row_stride) {
      record(word, b, p);
      continue;
    }
    const int64_t e = block_table[(int64_t)b * bt_row_stride + p];
    if (e < 0 || e >= num_pages) record(word, b, p);
  }
}

constexpr int kCheckBlocks = 16;

mla_status error_word(unsigned long long** word) {
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_error_word));
  if (e != hipSuccess)
    return fail(MLA_ERR_DEVICE, std::string("debug check: hipGetSymbolAddress: ") +
                                    hipGetErrorString(e));
  *word = static_cast<unsigned long long*>(p);
  return MLA_OK;
}

// Reads the word back after the check kernel; PRECONDITION with `what` and
// the first (request, index) if it was set.
mla_status read_word(const char* who, const char* what, const char* index_name,
                     unsigned long long* word, hipStream_t stream) {
  const mla_status launched = check_launch(who);
  if (launched != MLA_OK) return launched;
  unsigned long long v = kNone;
  hipError_t e = hipMemcpyAsync(&v, word, sizeof(v), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess)
    return fail(MLA_ERR_DEVICE, std::string(who) + ": debug check: " + hipGetErrorString(e));
  if (v == kNone) return MLA_OK;
  return fail(MLA_ERR_PRECONDITION, std::string(who) + ": " + what + " (first at request " +
                                        std::to_string(v >> 32) + ", " + index_name + " " +
                                        std::to_string(v & 0xffffffffu) + ")");
}

}  // namespace

mla_status debug_check_page_aligned(const char* who, const int32_t* req_to_token,
                                    int32_t r2t_rows, int64_t r2t_row_stride,
                                    const int32_t* req_pool_indices, const int32_t* seq_lens,
                                    int32_t bs, const int32_t* block_table,
                                    int32_t bt_row_stride, hipStream_t stream) {
  unsigned long long* word = nullptr;
  mla_status st = error_word(&word);
  if (st != MLA_OK) return st;
  hipLaunchKernelGGL(reset_word, dim3(1), dim3(1), 0, stream, word);
  hipLaunchKernelGGL(page_aligned_kernel, dim3(kCheckBlocks, bs), dim3(256), 0, stream,
                     req_to_token, r2t_rows, r2t_row_stride, req_pool_indices, seq_lens,
                     block_table, bt_row_stride, word);
  return read_word(who,
                   "a token's slot is not where its page's block-table entry puts it (slots not "
                   "page-aligned, or the table narrower than the request)",
                   "token", word, stream);
}

mla_status debug_check_table_entries(const char* who, const int32_t* block_table,
                                     int32_t bt_row_stride, const int32_t* seq_lens, int32_t bs,
                                     int64_t num_pages, hipStream_t stream) {
  unsigned long long* word = nullptr;
  mla_status st = error_word(&word);
  if (st != MLA_OK) return st;
  hipLaunchKernelGGL(reset_word, dim3(1), dim3(1), 0, stream, word);
  hipLaunchKernelGGL(table_entries_kernel, dim3(kCheckBlocks, bs), dim3(256), 0, stream,
                     block_table, bt_row_stride, seq_lens, num_pages, word);
  return read_word(who, "a block-table entry the decode reads is past the table or the pool",
                   "page", word, stream);
}

}  // namespace mla
