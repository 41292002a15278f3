// Internal helpers shared by the library's translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "mla_decode.h"

namespace mla {

constexpr int kPage = MLA_PAGE_SIZE;      // tokens per page
constexpr int kD = MLA_LATENT_DIM;        // latent row width (q/k)
constexpr int kDv = MLA_V_DIM;            // value width (first kDv columns)

// Records the error text for mla_last_error_message and returns the status.
mla_status fail(mla_status st, const std::string& msg);
// Clears the thread's error text and returns MLA_OK.
mla_status ok();
// Maps the result of hipGetLastError after a launch to a status.
mla_status check_launch(const char* what);
// True for a finite x >= 0.  Defined in abi.hip, which keeps IEEE NaN
// semantics (the decode kernel's file is compiled without them).
bool finite_nonneg(float x);

// Launch log: with the environment variable MLA_TRACE set (and not "0"),
// every launching entry point writes one line to stderr: the entry point, its
// sizes, grid and stream.  Read once per process.
bool trace_on();
void trace(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

#ifdef MLA_DEBUG
// Debug-build precondition checks (debug_checks.hip); each synchronises the
// stream and returns MLA_ERR_PRECONDITION naming the first violation.
mla_status debug_check_page_aligned(const char* who, const int32_t* req_to_token,
                                    int32_t r2t_rows, int64_t r2t_row_stride,
                                    const int32_t* req_pool_indices, const int32_t* seq_lens,
                                    int32_t bs, const int32_t* block_table,
                                    int32_t bt_row_stride, hipStream_t stream);
mla_status debug_check_table_entries(const char* who, const int32_t* block_table,
                                     int32_t bt_row_stride, const int32_t* seq_lens, int32_t bs,
                                     int64_t num_pages, hipStream_t stream);
#endif

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace mla
