// mla_decode_static: mla_decode followed by mla_merge_states, with the split
// pieces' partial (o, lse) states kept in a workspace that lives in the
// library's own device memory, so that the call allocates nothing.
//
// The workspace is a file-scope device array.  Its address on a device is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and kept; every later call on the device passes that address to the decode
// and merge kernels.  The array's name itself is never handed to a kernel or
// a copy: on the host it only stands for the symbol.
#include <mutex>
#include <string>

#include "common.h"

namespace mla {
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // MLA_STATIC_WORKSPACE_BYTES
static_assert(kScratchBytes == MLA_STATIC_WORKSPACE_BYTES, "header and library agree");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
hipError_t g_scratch_err[kMaxDevices] = {};
std::once_flag g_scratch_once[kMaxDevices];

// The workspace address on the current device (nullptr and a status on
// failure).
mla_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(MLA_ERR_DEVICE, std::string("mla_decode_static: hipGetDevice: ") +
                                    hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_static: device index above 63");
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g_scratch_err[dev] == hipSuccess) g_scratch[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch[dev])
    return fail(MLA_ERR_DEVICE, std::string("mla_decode_static: hipGetSymbolAddress: ") +
                                    hipGetErrorString(g_scratch_err[dev]));
  *ptr = g_scratch[dev];
  return MLA_OK;
}

}  // namespace
}  // namespace mla

extern "C" mla_status mla_decode_static(const void* q, int32_t bs, int32_t q_len,
                                        int32_t num_heads, const void* kv_cache, int32_t kv_dtype,
                                        int64_t num_pages, const int32_t* block_table,
                                        int32_t bt_row_stride, const int32_t* seq_lens,
                                        const int32_t* tile_plan, int32_t num_parts,
                                        const int32_t* split_indptr, float softmax_scale,
                                        int32_t causal, const float* kv_descale, void* out,
                                        float* lse, hipStream_t stream) {
  using namespace mla;
  if (bs <= 0 || q_len <= 0 || num_heads <= 0 || num_parts <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_static: sizes must be positive");
  const int64_t rows = (int64_t)q_len * num_heads;
  const int64_t slots = (int64_t)bs + num_parts;
  if (rows > MLA_MAX_ROWS_PER_REQ)
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_static: q_len*num_heads must be in 1..512");
  const size_t o_bytes = (size_t)slots * (size_t)rows * MLA_V_DIM * sizeof(uint16_t);
  const size_t need = o_bytes + (size_t)slots * (size_t)rows * sizeof(float);
  if (need > kScratchBytes)
    return fail(MLA_ERR_CAPACITY,
                "mla_decode_static: (bs + num_parts) * rows * 1028 bytes = " +
                    std::to_string(need) + " exceeds the static workspace of " +
                    std::to_string(kScratchBytes) + " bytes");
  void* base = nullptr;
  const mla_status st = scratch_of_current_device(&base);
  if (st != MLA_OK) return st;
  uint8_t* const ws = static_cast<uint8_t*>(base);
  void* const partial_o = ws;                                    // bf16 [slots, rows, 512]
  float* const partial_lse = reinterpret_cast<float*>(ws + o_bytes);  // fp32 [slots, rows]
  // Every slot the merge reads is one the decode writes in this call (a
  // plan's pieces), so the workspace needs no clearing.
  mla_status s = mla_decode(q, bs, q_len, num_heads, kv_cache, kv_dtype, num_pages, block_table,
                            bt_row_stride, seq_lens, tile_plan, num_parts, split_indptr,
                            softmax_scale, causal, kv_descale, partial_o, partial_lse,
                            (int32_t)slots, out, lse, stream);
  if (s != MLA_OK) return s;
  return mla_merge_states(partial_o, partial_lse, (int32_t)slots, split_indptr, bs, (int32_t)rows,
                          MLA_V_DIM, out, lse, stream);
}
