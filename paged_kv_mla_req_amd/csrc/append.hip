// KV append: store the new tokens' latent rows into their pool slots.
//
// What it computes (FlashMLA backend page, forward_decode and the
// target-verify branch of forward_extend: token_to_kv_pool.set_kv_buffer with
// cache_loc = forward_batch.out_cache_loc, before the attention call): for
// each new token i, latent row k[i] (576 wide; in MLA V is its first 512
// columns, so nothing else is stored) goes to slot s = out_cache_loc[i], i.e.
// row s % 64 of page s / 64 of the pool [num_pages, 64, 576] that the decode
// reads.  For an fp8 cache the stored byte is the OCP e4m3fn value nearest to
// k / scale (ties to even, saturating at 448), the quotient rounded to fp32;
// the decode multiplies the byte's value by the same per-tensor scale.
//
// The same kernel, with row i stored to row i, quantises the query for the
// cache's fp8 branch (scaled_fp8_quant(q, q_scale) with q_scale = k_scale in
// forward_decode): code = e4m3fn(q / q_scale), rounded and saturated as the
// cache bytes are.
//
// How (gfx950): the work is pure data movement, bound by HBM (large appends)
// or launch latency (one token per request).  One thread moves one 16-byte
// chunk of 8 bf16 values; the 72 chunks of a row are consecutive threads, so
// each row is read and each slot written as one contiguous run.
#include "common.h"

namespace mla {

constexpr int kAppendThreads = 256;
constexpr int kAppendChunks = kD / 8;  // 72 chunks of 8 bf16 per latent row

// fp32 -> e4m3fn code, nearest value with ties to even, |x| > 448 saturating
// to 448, NaN to S.1111.111.  Written from the format: normal values keep 3
// mantissa bits, rounded on the fp32 bit pattern (the carry moves into the
// exponent when the mantissa overflows); below 2^-6 the grid is m * 2^-9,
// m = 0..7 (m = 8 is the smallest normal code, 0x08).
__device__ __forceinline__ uint32_t e4m3fn_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;            // NaN
  if (a > 0x43e00000u) return sign | 0x7eu;            // above 448, infinity included
  if (a < 0x3c800000u) {                                // below 2^-6
    const float m = __uint_as_float(a) * 512.0f;        // exact: a power-of-two scaling
    return sign | (uint32_t)__builtin_rintf(m);         // ties to even
  }
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);   // round to 3 mantissa bits
  return sign | ((r >> 20) - (120u << 3));              // rebias: 127 - 7 = 120
}

template <bool kFp8>
__global__ __launch_bounds__(kAppendThreads) void set_kv_kernel(
    const uint16_t* __restrict__ k, int64_t k_row_stride, const int64_t* __restrict__ slots,
    int32_t n, uint8_t* __restrict__ kv, int64_t num_slots, const float* __restrict__ kv_scale) {
  const int64_t g = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
  const int64_t row = g / kAppendChunks;
  const int c = (int)(g - row * kAppendChunks);
  if (row >= n) return;
  const int64_t s = slots ? slots[row] : row;   // no slot list: row i goes to row i
  if (s < 0 || s >= num_slots) return;   // a slot outside the pool is never written
  const uint4 v = *reinterpret_cast<const uint4*>(k + row * k_row_stride + c * 8);
  if constexpr (!kFp8) {
    *reinterpret_cast<uint4*>(kv + s * (kD * 2) + c * 16) = v;
  } else {
    const float d = *kv_scale;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(w[i] << 16);          // element 2i
      const float hi = __uint_as_float(w[i] & 0xffff0000u);  // element 2i + 1
      const uint32_t pair = e4m3fn_code(lo / d) | (e4m3fn_code(hi / d) << 8);
      packed[i >> 1] |= pair << (16 * (i & 1));
    }
    *reinterpret_cast<uint2*>(kv + s * kD + c * 8) = make_uint2(packed[0], packed[1]);
  }
}

}  // namespace mla

extern "C" mla_status mla_set_kv_buffer(const void* k, int64_t k_row_stride,
                                        const int64_t* out_cache_loc, int32_t num_tokens,
                                        void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                                        const float* kv_scale, hipStream_t stream) {
  using namespace mla;
  // With no tokens, k and out_cache_loc are never read and may be NULL.
  if (!kv_cache || (num_tokens > 0 && (!k || !out_cache_loc)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_set_kv_buffer: null pointer");
  if (num_tokens < 0 || num_pages <= 0 || k_row_stride < kD)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "mla_set_kv_buffer: need num_tokens >= 0, num_pages > 0, k_row_stride >= 576");
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, "mla_set_kv_buffer: unknown kv_dtype");
  const bool fp8 = kv_dtype == MLA_KV_FP8_E4M3;
  if (fp8 && !kv_scale)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_set_kv_buffer: fp8 cache needs kv_scale");
  if ((reinterpret_cast<uintptr_t>(k) & 15u) || (k_row_stride & 7) ||
      (reinterpret_cast<uintptr_t>(kv_cache) & 15u))
    return fail(MLA_ERR_UNSUPPORTED,
                "mla_set_kv_buffer: k and kv_cache must be 16-byte aligned, k_row_stride a "
                "multiple of 8");
  if (num_pages > INT64_MAX / (kPage * kD * 2))
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_set_kv_buffer: num_pages too large");
  if (num_tokens == 0) return ok();
  const int64_t threads = (int64_t)num_tokens * kAppendChunks;
  const unsigned blocks = (unsigned)((threads + kAppendThreads - 1) / kAppendThreads);
  const int64_t num_slots = num_pages * kPage;
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  uint8_t* dst = static_cast<uint8_t*>(kv_cache);
  trace("mla_set_kv_buffer: tokens %d kv_dtype %d pages %lld grid %u stream %p", num_tokens,
        kv_dtype, (long long)num_pages, blocks, (void*)stream);
  if (fp8)
    set_kv_kernel<true><<<blocks, kAppendThreads, 0, stream>>>(kk, k_row_stride, out_cache_loc,
                                                               num_tokens, dst, num_slots, kv_scale);
  else
    set_kv_kernel<false><<<blocks, kAppendThreads, 0, stream>>>(kk, k_row_stride, out_cache_loc,
                                                                num_tokens, dst, num_slots, nullptr);
  return check_launch("mla_set_kv_buffer");
}

extern "C" mla_status mla_quantize_q_fp8(const void* q, int64_t q_row_stride, int64_t num_rows,
                                         const float* q_scale, void* q_fp8, hipStream_t stream) {
  using namespace mla;
  if (!q_scale || !q_fp8 || (num_rows > 0 && !q))
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_quantize_q_fp8: null pointer");
  if (num_rows < 0 || q_row_stride < kD)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "mla_quantize_q_fp8: need num_rows >= 0 and q_row_stride >= 576");
  if ((reinterpret_cast<uintptr_t>(q) & 15u) || (q_row_stride & 7) ||
      (reinterpret_cast<uintptr_t>(q_fp8) & 7u))
    return fail(MLA_ERR_UNSUPPORTED,
                "mla_quantize_q_fp8: q must be 16-byte aligned, q_row_stride a multiple of 8, "
                "q_fp8 8-byte aligned");
  if (num_rows > INT32_MAX)
    return fail(MLA_ERR_UNSUPPORTED, "mla_quantize_q_fp8: more than 2^31 - 1 rows");
  if (num_rows == 0) return ok();
  const int64_t threads = num_rows * kAppendChunks;
  const unsigned blocks = (unsigned)((threads + kAppendThreads - 1) / kAppendThreads);
  trace("mla_quantize_q_fp8: rows %lld grid %u stream %p", (long long)num_rows, blocks,
        (void*)stream);
  set_kv_kernel<true><<<blocks, kAppendThreads, 0, stream>>>(
      static_cast<const uint16_t*>(q), q_row_stride, nullptr, (int32_t)num_rows,
      static_cast<uint8_t*>(q_fp8), num_rows, q_scale);
  return check_launch("mla_quantize_q_fp8");
}
