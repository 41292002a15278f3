// Host-side driver of the C ABI for the sanitizer build (tests/test_sanitize.py
// links it with the library sources compiled with -fsanitize=address and
// -fsanitize=undefined on the host side).  Every call below fails argument
// validation before it would touch a device, or is a host helper, so the
// driver runs without a GPU; it checks each status and error text and exits
// non-zero on the first mismatch.  Two threads make failing calls at once, so
// that each thread's error text is exercised under the sanitizers.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>

#include "mla_decode.h"

namespace {

std::atomic<int> g_failures{0};
std::atomic<int> g_checks{0};

void expect(const char* what, mla_status got, mla_status want, const char* prefix) {
  ++g_checks;
  const char* msg = mla_last_error_message();
  if (got != want || (want != MLA_OK && std::strncmp(msg, prefix, std::strlen(prefix)) != 0)) {
    std::printf("FAIL %s: status %d (want %d), message \"%s\"\n", what, got, want, msg);
    ++g_failures;
  }
}

// never dereferenced: every call that receives them fails validation first
alignas(64) int32_t g_i32[64];
alignas(64) float g_f32[64];
alignas(64) int64_t g_i64[64];
void* const F = g_i32;
float* const FF = g_f32;
int32_t* const FI = g_i32;

mla_status decode(const void* q, int bs, int q_len, int heads, int dtype, float scale,
                  const float* descale, int parts, int slots) {
  return mla_decode(q, bs, q_len, heads, F, dtype, 8, FI, 3, FI, FI, parts, FI, scale, 1, descale,
                    F, FF, slots, F, nullptr, nullptr);
}

void decode_cases() {
  const mla_status I = MLA_ERR_INVALID_ARGUMENT, U = MLA_ERR_UNSUPPORTED, C = MLA_ERR_CAPACITY;
  expect("decode null q", decode(nullptr, 2, 1, 16, 0, 0.1f, nullptr, 4, 6), I, "mla_decode");
  expect("decode bs 0", decode(F, 0, 1, 16, 0, 0.1f, nullptr, 4, 6), I, "mla_decode");
  expect("decode heads -1", decode(F, 2, 1, -1, 0, 0.1f, nullptr, 4, 6), I, "mla_decode");
  expect("decode scale nan", decode(F, 2, 1, 16, 0, __builtin_nanf(""), nullptr, 4, 6), I,
         "mla_decode");
  expect("decode scale inf", decode(F, 2, 1, 16, 0, __builtin_inff(), nullptr, 4, 6), I,
         "mla_decode");
  expect("decode scale < 0", decode(F, 2, 1, 16, 0, -0.5f, nullptr, 4, 6), I, "mla_decode");
  expect("decode dtype 7", decode(F, 2, 1, 16, 7, 0.1f, nullptr, 4, 6), U, "mla_decode");
  expect("decode fp8 no descale", decode(F, 2, 1, 16, 1, 0.1f, nullptr, 4, 6), I, "mla_decode");
  expect("decode rows 513", decode(F, 2, 1, 513, 0, 0.1f, nullptr, 4, 6), U, "mla_decode");
  expect("decode rows 640", decode(F, 2, 5, 128, 0, 0.1f, nullptr, 4, 6), U, "mla_decode");
  expect("decode slots", decode(F, 2, 1, 16, 0, 0.1f, nullptr, 4, 5), C, "mla_decode");
  expect("decode parts", decode(F, 2, 1, 16, 0, 0.1f, nullptr, 65537, 70000), C, "mla_decode");
  expect("decode_q8 no q_descale",
         mla_decode_q8(F, nullptr, 2, 1, 16, F, 8, FI, 3, FI, FI, 4, FI, 0.1f, 1, FF, F, FF, 6, F,
                       nullptr, nullptr),
         I, "mla_decode_q8");
  expect("decode_q8 no kv_descale",
         mla_decode_q8(F, FF, 2, 1, 16, F, 8, FI, 3, FI, FI, 4, FI, 0.1f, 1, nullptr, F, FF, 6, F,
                       nullptr, nullptr),
         I, "mla_decode_q8");
  expect("decode_static bs 0",
         mla_decode_static(F, 0, 1, 16, F, 0, 8, FI, 3, FI, FI, 4, FI, 0.1f, 1, nullptr, F,
                           nullptr, nullptr),
         I, "mla_decode_static");
  expect("decode_static capacity",
         mla_decode_static(F, 512, 1, 128, F, 0, 8, FI, 3, FI, FI, 256, FI, 0.1f, 1, nullptr, F,
                           nullptr, nullptr),
         C, "mla_decode_static");
}

void table_and_plan_cases() {
  const mla_status I = MLA_ERR_INVALID_ARGUMENT, U = MLA_ERR_UNSUPPORTED, C = MLA_ERR_CAPACITY;
  expect("table null", mla_build_block_table(nullptr, 4, 64, FI, FI, 2, 64, FI, 3, -1, -1, nullptr),
         I, "mla_build_block_table");
  expect("table bs 0", mla_build_block_table(FI, 4, 64, FI, FI, 0, 64, FI, 3, -1, -1, nullptr), I,
         "mla_build_block_table");
  expect("table page 32", mla_build_block_table(FI, 4, 64, FI, FI, 2, 32, FI, 3, -1, -1, nullptr),
         U, "mla_build_block_table");
  expect("table narrow hint",
         mla_build_block_table(FI, 4, 1024, FI, FI, 2, 64, FI, 3, -1, 1000, nullptr), C,
         "mla_build_block_table");
  expect("table short r2t", mla_build_block_table(FI, 4, 64, FI, FI, 2, 64, FI, 30, -1, 1000, nullptr),
         C, "mla_build_block_table");
  expect("plan null", mla_plan_splits(nullptr, 2, 16, 4, 0, FI, FI, nullptr), I, "mla_plan_splits");
  expect("plan parts 0", mla_plan_splits(FI, 2, 16, 0, 0, FI, FI, nullptr), I, "mla_plan_splits");
  expect("plan rows 600", mla_plan_splits(FI, 2, 600, 4, 0, FI, FI, nullptr), U, "mla_plan_splits");
  expect("fused null",
         mla_build_table_and_plan(nullptr, 4, 64, FI, FI, 2, 64, FI, 3, -1, -1, 16, 4, 0, FI, FI,
                                  nullptr),
         I, "mla_build_table_and_plan");
  expect("fixed tile 0", mla_plan_fixed_splits(FI, 2, 0, 8, -1, FI, FI, nullptr), I,
         "mla_plan_fixed_splits");
  expect("fixed bound", mla_plan_fixed_splits(FI, 2, 32, 1, 4096, FI, FI, nullptr), C,
         "mla_plan_fixed_splits");
  expect("merge null", mla_merge_states(nullptr, FF, 4, FI, 2, 16, 512, F, FF, nullptr), I,
         "mla_merge_states");
  expect("merge dv", mla_merge_states(F, FF, 4, FI, 2, 16, 256, F, FF, nullptr), U,
         "mla_merge_states");
  expect("merge misaligned",
         mla_merge_states(reinterpret_cast<char*>(F) + 4, FF, 4, FI, 2, 16, 512, F, FF, nullptr), U,
         "mla_merge_states");
  expect("append null", mla_set_kv_buffer(nullptr, 576, g_i64, 2, F, 0, 8, nullptr, nullptr), I,
         "mla_set_kv_buffer");
  expect("append stride", mla_set_kv_buffer(F, 500, g_i64, 2, F, 0, 8, nullptr, nullptr), I,
         "mla_set_kv_buffer");
  expect("append fp8 no scale", mla_set_kv_buffer(F, 576, g_i64, 2, F, 1, 8, nullptr, nullptr), I,
         "mla_set_kv_buffer");
  expect("append empty", mla_set_kv_buffer(nullptr, 576, nullptr, 0, F, 0, 8, nullptr, nullptr),
         MLA_OK, "");
  expect("quantize rows -1", mla_quantize_q_fp8(F, 576, -1, FF, F, nullptr), I,
         "mla_quantize_q_fp8");
  expect("quantize misaligned",
         mla_quantize_q_fp8(reinterpret_cast<char*>(F) + 2, 576, 4, FF, F, nullptr), U,
         "mla_quantize_q_fp8");
  expect("quantize empty", mla_quantize_q_fp8(nullptr, 576, 0, FF, F, nullptr), MLA_OK, "");
}

void helper_cases() {
  ++g_checks;
  if (mla_abi_version() != MLA_ABI_VERSION) ++g_failures;
  for (int s = -1; s <= 6; ++s) {
    ++g_checks;
    const char* t = mla_status_string(s);
    if (!t || !*t) ++g_failures;
  }
  ++g_checks;
  if (mla_max_total_splits(64, 256) != 320 || mla_max_total_splits(-1, 2) != -1) ++g_failures;
  ++g_checks;
  if (mla_workspace_bytes(64, 128, 256) != (size_t)320 * 128 * 1028 ||
      mla_workspace_bytes(-1, 1, 1) != 0 || mla_partial_bytes(2, 3, 4) != mla_workspace_bytes(2, 3, 4))
    ++g_failures;
  ++g_checks;
  if (mla_fixed_split_parts_bound(64, 8192, 32) != 64 * 4 ||
      mla_fixed_split_parts_bound(1, 4096, 0) != -1 ||
      mla_fixed_split_parts_bound(65535, 0x7fffffff, 1) != 0x7fffffff)
    ++g_failures;
  ++g_checks;
  if (mla_decode_time_next_launch(nullptr, nullptr) != MLA_OK) ++g_failures;
  (void)mla_device_num_cus();  // -1 without a device, the CU count with one
}

}  // namespace

int main() {
  helper_cases();
  std::thread t1([] {
    for (int i = 0; i < 200; ++i) decode_cases();
  });
  std::thread t2([] {
    for (int i = 0; i < 200; ++i) table_and_plan_cases();
  });
  t1.join();
  t2.join();
  decode_cases();
  table_and_plan_cases();
  std::printf("%d checks, %d failures\n", g_checks.load(), g_failures.load());
  return g_failures == 0 ? 0 : 1;
}
