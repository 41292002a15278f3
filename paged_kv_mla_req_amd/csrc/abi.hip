// Status codes, error text, the launch log and host helpers of the C ABI.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "common.h"

namespace mla {

static thread_local std::string g_last_error;

mla_status fail(mla_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

mla_status ok() {
  g_last_error.clear();
  return MLA_OK;
}

bool finite_nonneg(float x) { return std::isfinite(x) && x >= 0.f; }

bool trace_on() {
  static const bool on = [] {
    const char* e = std::getenv("MLA_TRACE");
    return e && *e && std::strcmp(e, "0") != 0;
  }();
  return on;
}

void trace(const char* fmt, ...) {
  if (!trace_on()) return;
  char line[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(line, sizeof(line), fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[mla] %s\n", line);
}

mla_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(MLA_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
  return ok();
}

}  // namespace mla

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(int32_t status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported";
    case MLA_ERR_CAPACITY: return "capacity exceeded";
    case MLA_ERR_PRECONDITION: return "precondition violated";
    case MLA_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* mla_last_error_message(void) { return mla::g_last_error.c_str(); }

int32_t mla_max_total_splits(int32_t bs, int32_t num_parts) {
  if (bs < 0 || num_parts < 0) return -1;
  return bs + num_parts;
}

size_t mla_workspace_bytes(int32_t bs, int32_t rows_per_req, int32_t num_parts) {
  if (bs < 0 || num_parts < 0 || rows_per_req < 0) return 0;
  const size_t slots = (size_t)bs + (size_t)num_parts;
  // bf16 partial o [slots, rows, 512], then fp32 partial lse [slots, rows]
  return slots * (size_t)rows_per_req * (MLA_V_DIM * sizeof(uint16_t) + sizeof(float));
}

size_t mla_partial_bytes(int32_t bs, int32_t rows_per_req, int32_t num_parts) {
  return mla_workspace_bytes(bs, rows_per_req, num_parts);
}

int32_t mla_device_num_cus(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cus;
}

}  // extern "C"
