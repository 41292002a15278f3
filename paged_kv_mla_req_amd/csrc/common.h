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

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace mla
