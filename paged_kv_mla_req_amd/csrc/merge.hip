// Exact merge of partial attention states.
//
// The FlashInfer backend page computes attention over two disjoint key sets
// (ragged new tokens, paged prefix), each returning (o, lse), and combines
// them with merge_state; the FlashMLA page returns lse so that decode
// context-parallel ranks can correct their outputs the same way.  This kernel
// does the k-way form for every request whose keys mla_decode split into k
// pieces:  LSE = M + ln sum_k exp(lse_k - M),  o = sum_k exp(lse_k - LSE) o_k.
//
// One wave per (request, row): each lane owns 8 of the 512 value columns (two
// 16-byte loads per piece, so a piece's row is read fully coalesced), with the
// rows of eight pieces in flight at a time; for up to 64 pieces the lanes take
// one piece's lse each (wave max and sum) while the first rows are already
// loading, so a row costs one memory round trip.  Pure HBM streaming; no MFMA.
#include "common.h"

namespace mla {

constexpr int kMergeWaves = 4;
constexpr int kMergeBatch = 8;  // pieces whose rows are loaded together

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = fmaxf(x, __shfl_xor(x, d, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

__global__ void __launch_bounds__(64 * kMergeWaves)
merge_states_kernel(const float* __restrict__ partial_o, const float* __restrict__ partial_lse,
                    const int32_t* __restrict__ split_indptr, int bs, int rows,
                    uint16_t* __restrict__ out, float* __restrict__ lse_out) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (gw >= (int64_t)bs * rows) return;
  const int b = (int)(gw / rows);
  const int r = (int)(gw - (int64_t)b * rows);
  const int k0 = split_indptr[b];
  const int k = split_indptr[b + 1] - k0;
  if (k == 1) return;  // already final

  float4 acc0 = make_float4(0.f, 0.f, 0.f, 0.f), acc1 = acc0;
  float LSE = -INFINITY;
  if (k > 1 && k <= 64) {
    // One round trip: lane s takes piece s's lse while the rows of the first
    // kMergeBatch pieces are already on their way (they do not depend on it).
    const float l = lane < k ? partial_lse[(int64_t)(k0 + lane) * rows + r] : -INFINITY;
    float4 x0[kMergeBatch], x1[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      x0[j] = x1[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < k) {
        const float4* src =
            reinterpret_cast<const float4*>(partial_o + ((int64_t)(k0 + j) * rows + r) * kDv) +
            lane * 2;
        x0[j] = src[0];
        x1[j] = src[1];
      }
    }
    const float M = wave_max(l);
    if (M != -INFINITY) {
      LSE = M + __logf(wave_sum(l == -INFINITY ? 0.f : __expf(l - M)));
      const float wl = l == -INFINITY ? 0.f : __expf(l - LSE);  // piece `lane`'s weight
      for (int s0 = 0; s0 < k; s0 += kMergeBatch) {
        if (s0 > 0) {
#pragma unroll
          for (int j = 0; j < kMergeBatch; ++j) {
            x0[j] = x1[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (s0 + j < k) {
              const float4* src = reinterpret_cast<const float4*>(
                                      partial_o + ((int64_t)(k0 + s0 + j) * rows + r) * kDv) +
                                  lane * 2;
              x0[j] = src[0];
              x1[j] = src[1];
            }
          }
        }
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          const float w = __shfl(wl, (s0 + j) & 63, 64);  // 0 past the last piece
          acc0.x += w * x0[j].x; acc0.y += w * x0[j].y;
          acc0.z += w * x0[j].z; acc0.w += w * x0[j].w;
          acc1.x += w * x1[j].x; acc1.y += w * x1[j].y;
          acc1.z += w * x1[j].z; acc1.w += w * x1[j].w;
        }
      }
    }
  } else if (k > 64) {
    // M and the sum of exp(lse - M): the lanes take the pieces' lse values
    float m = -INFINITY;
    for (int s = lane; s < k; s += 64) m = fmaxf(m, partial_lse[(int64_t)(k0 + s) * rows + r]);
    const float M = wave_max(m);
    if (M != -INFINITY) {
      float t = 0.f;
      for (int s = lane; s < k; s += 64) {
        const float l = partial_lse[(int64_t)(k0 + s) * rows + r];
        t += (l == -INFINITY) ? 0.f : __expf(l - M);
      }
      LSE = M + __logf(wave_sum(t));
      // o = sum_k exp(lse_k - LSE) o_k, kMergeBatch rows in flight at a time
      for (int s0 = 0; s0 < k; s0 += kMergeBatch) {
        float4 x0[kMergeBatch], x1[kMergeBatch];
        float w[kMergeBatch];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          const int s = s0 + j;
          w[j] = 0.f;
          x0[j] = x1[j] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (s < k) {
            const float l = partial_lse[(int64_t)(k0 + s) * rows + r];
            w[j] = (l == -INFINITY) ? 0.f : __expf(l - LSE);
            const float4* src = reinterpret_cast<const float4*>(
                                    partial_o + ((int64_t)(k0 + s) * rows + r) * kDv) + lane * 2;
            x0[j] = src[0];
            x1[j] = src[1];
          }
        }
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          acc0.x += w[j] * x0[j].x; acc0.y += w[j] * x0[j].y;
          acc0.z += w[j] * x0[j].z; acc0.w += w[j] * x0[j].w;
          acc1.x += w[j] * x1[j].x; acc1.y += w[j] * x1[j].y;
          acc1.z += w[j] * x1[j].z; acc1.w += w[j] * x1[j].w;
        }
      }
    }
  }
  uint4 packed;
  packed.x = (uint32_t)f32_to_bf16(acc0.x) | ((uint32_t)f32_to_bf16(acc0.y) << 16);
  packed.y = (uint32_t)f32_to_bf16(acc0.z) | ((uint32_t)f32_to_bf16(acc0.w) << 16);
  packed.z = (uint32_t)f32_to_bf16(acc1.x) | ((uint32_t)f32_to_bf16(acc1.y) << 16);
  packed.w = (uint32_t)f32_to_bf16(acc1.z) | ((uint32_t)f32_to_bf16(acc1.w) << 16);
  reinterpret_cast<uint4*>(out + ((int64_t)b * rows + r) * kDv)[lane] = packed;
  if (lse_out && lane == 0) lse_out[(int64_t)b * rows + r] = LSE;
}

}  // namespace mla

extern "C" mla_status mla_merge_states(const float* partial_o, const float* partial_lse,
                                       const int32_t* split_indptr, int32_t bs,
                                       int32_t rows_per_req, void* out, float* lse,
                                       hipStream_t stream) {
  using namespace mla;
  if (!partial_o || !partial_lse || !split_indptr || !out)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_merge_states: null pointer");
  if (bs <= 0) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_merge_states: bs must be positive");
  if (rows_per_req < 1 || rows_per_req > MLA_MAX_ROWS_PER_REQ)
    return fail(MLA_ERR_UNSUPPORTED, "mla_merge_states: rows_per_req must be in 1..512");
  const int64_t waves = (int64_t)bs * rows_per_req;
  const int64_t blocks = (waves + kMergeWaves - 1) / kMergeWaves;
  if (blocks > 0x7fffffff) return fail(MLA_ERR_UNSUPPORTED, "mla_merge_states: too many rows");
  hipLaunchKernelGGL(merge_states_kernel, dim3((unsigned)blocks), dim3(64 * kMergeWaves), 0,
                     stream, partial_o, partial_lse, split_indptr, bs, rows_per_req,
                     reinterpret_cast<uint16_t*>(out), lse);
  return check_launch("mla_merge_states");
}
