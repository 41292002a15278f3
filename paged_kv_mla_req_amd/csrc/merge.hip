// Exact merge of partial attention states.
//
// The FlashInfer backend page computes attention over two disjoint key sets
// (ragged new tokens, paged prefix), each returning (o, lse), and combines
// them with merge_state; the FlashMLA page returns lse so that decode
// context-parallel ranks can correct their outputs the same way.  This kernel
// does the k-way form for every request whose keys mla_decode split into k
// pieces:  LSE = M + ln sum_k exp(lse_k - M),  o = sum_k exp(lse_k - LSE) o_k.
//
// A piece's o is stored in bf16 (normalised by its own row sum) and its lse in
// fp32.  One wave per (request, row): each lane owns 8 of the 512 value
// columns, one 16-byte load per piece, so a piece's row is one coalesced
// 1 KiB read, with the rows of eight pieces in flight at a time (63 VGPRs: eight
// waves per SIMD, so the whole DeepSeek-V3-shaped batch is resident at once); for up to
// 64 pieces the lanes take one piece's lse each (wave max and sum) while the
// first rows are already loading, so a row costs one memory round trip.
// Pure HBM streaming; no MFMA.
#include "common.h"

namespace mla {

constexpr int kMergeWaves = 4;
constexpr int kXcdsMerge = 8;  // accelerator dies, each with its own L2
constexpr int kMergeBatch = 8;   // pieces whose rows are loaded together

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

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// acc[0..7] += w * (8 bf16 values in x)
__device__ __forceinline__ void fma8(float (&acc)[8], float w, const uint4& x) {
  acc[0] += w * bf16_lo(x.x);
  acc[1] += w * bf16_hi(x.x);
  acc[2] += w * bf16_lo(x.y);
  acc[3] += w * bf16_hi(x.y);
  acc[4] += w * bf16_lo(x.z);
  acc[5] += w * bf16_hi(x.z);
  acc[6] += w * bf16_lo(x.w);
  acc[7] += w * bf16_hi(x.w);
}

__global__ void __launch_bounds__(64 * kMergeWaves)
merge_states_kernel(const uint16_t* __restrict__ partial_o, const float* __restrict__ partial_lse,
                    int partial_slots, const int32_t* __restrict__ split_indptr, int bs,
                    int rows, uint16_t* __restrict__ out, float* __restrict__ lse_out) {
  const int lane = threadIdx.x & 63;
  // Work-groups go to the dies round robin (work-group i to die i % 8).  The
  // decode leaves each die a contiguous run of parts, i.e. of requests, so
  // the merge gives each die a contiguous run of rows as well: most of a
  // request's partial rows are then read on the die that wrote them.
  const int64_t nblk = gridDim.x, per = nblk / kXcdsMerge, extra = nblk % kXcdsMerge;
  const int64_t x = blockIdx.x % kXcdsMerge, j = blockIdx.x / kXcdsMerge;
  const int64_t blk = x * per + (x < extra ? x : extra) + j;
  const int64_t gw = blk * kMergeWaves + (threadIdx.x >> 6);
  if (gw >= (int64_t)bs * rows) return;
  const int b = (int)(gw / rows);
  const int r = (int)(gw - (int64_t)b * rows);
  const int k0 = split_indptr[b];
  const int k = split_indptr[b + 1] - k0;
  if (k == 1) return;  // already final

  // a piece whose slot lies outside the workspace is absent (weight 0)
  auto present = [&](int s) { return k0 + s >= 0 && k0 + s < partial_slots; };
  auto lse_of = [&](int s) {
    return present(s) ? partial_lse[(int64_t)(k0 + s) * rows + r] : -INFINITY;
  };
  auto row_of = [&](int s) {
    return present(s)
               ? reinterpret_cast<const uint4*>(partial_o + ((int64_t)(k0 + s) * rows + r) * kDv)[lane]
               : make_uint4(0, 0, 0, 0);
  };

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float LSE = -INFINITY;
  if (k > 1 && k <= 64) {
    // One round trip: lane s takes piece s's lse while the rows of the first
    // kMergeBatch pieces are already on their way (they do not depend on it).
    const float l = lane < k ? lse_of(lane) : -INFINITY;
    uint4 x[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) x[j] = j < k ? row_of(j) : make_uint4(0, 0, 0, 0);
    const float M = wave_max(l);
    if (M != -INFINITY) {
      LSE = M + __logf(wave_sum(l == -INFINITY ? 0.f : __expf(l - M)));
      const float wl = l == -INFINITY ? 0.f : __expf(l - LSE);  // piece `lane`'s weight
      for (int s0 = 0; s0 < k; s0 += kMergeBatch) {
        if (s0 > 0) {
#pragma unroll
          for (int j = 0; j < kMergeBatch; ++j)
            x[j] = s0 + j < k ? row_of(s0 + j) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          const float w = __shfl(wl, (s0 + j) & 63, 64);  // 0 past the last piece
          fma8(acc, w, x[j]);
        }
      }
    }
  } else if (k > 64) {
    // M and the sum of exp(lse - M): the lanes take the pieces' lse values
    float m = -INFINITY;
    for (int s = lane; s < k; s += 64) m = fmaxf(m, lse_of(s));
    const float M = wave_max(m);
    if (M != -INFINITY) {
      float t = 0.f;
      for (int s = lane; s < k; s += 64) {
        const float l = lse_of(s);
        t += (l == -INFINITY) ? 0.f : __expf(l - M);
      }
      LSE = M + __logf(wave_sum(t));
      // o = sum_k exp(lse_k - LSE) o_k, kMergeBatch rows in flight at a time
      for (int s0 = 0; s0 < k; s0 += kMergeBatch) {
        uint4 x[kMergeBatch];
        float w[kMergeBatch];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          const int s = s0 + j;
          w[j] = 0.f;
          x[j] = make_uint4(0, 0, 0, 0);
          if (s < k) {
            const float l = lse_of(s);
            w[j] = (l == -INFINITY) ? 0.f : __expf(l - LSE);
            x[j] = row_of(s);
          }
        }
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) fma8(acc, w[j], x[j]);
      }
    }
  }
  uint4 packed;
  packed.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
  packed.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
  packed.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
  packed.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
  reinterpret_cast<uint4*>(out + ((int64_t)b * rows + r) * kDv)[lane] = packed;
  if (lse_out && lane == 0) lse_out[(int64_t)b * rows + r] = LSE;
}

}  // namespace mla

extern "C" mla_status mla_merge_states(const void* partial_o, const float* partial_lse,
                                       int32_t partial_slots, const int32_t* split_indptr,
                                       int32_t bs, int32_t rows_per_req, int32_t dv, void* out,
                                       float* lse, hipStream_t stream) {
  using namespace mla;
  if (!partial_o || !partial_lse || !split_indptr || !out)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_merge_states: null pointer");
  if (bs <= 0) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_merge_states: bs must be positive");
  if (partial_slots < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_merge_states: partial_slots must be >= 0");
  if (rows_per_req < 1 || rows_per_req > MLA_MAX_ROWS_PER_REQ)
    return fail(MLA_ERR_UNSUPPORTED, "mla_merge_states: rows_per_req must be in 1..512");
  if (dv != MLA_V_DIM) return fail(MLA_ERR_UNSUPPORTED, "mla_merge_states: dv must be 512");
  if ((reinterpret_cast<uintptr_t>(partial_o) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(MLA_ERR_UNSUPPORTED, "mla_merge_states: partial_o and out must be 16-byte aligned");
  const int64_t waves = (int64_t)bs * rows_per_req;
  const int64_t blocks = (waves + kMergeWaves - 1) / kMergeWaves;
  if (blocks > 0x7fffffff) return fail(MLA_ERR_UNSUPPORTED, "mla_merge_states: too many rows");
  trace("mla_merge_states: bs %d rows %d slots %d grid %lld stream %p", bs, rows_per_req,
        partial_slots, (long long)blocks, (void*)stream);
  hipLaunchKernelGGL(merge_states_kernel, dim3((unsigned)blocks), dim3(64 * kMergeWaves), 0,
                     stream, reinterpret_cast<const uint16_t*>(partial_o), partial_lse,
                     partial_slots, split_indptr, bs, rows_per_req,
                     reinterpret_cast<uint16_t*>(out), lse);
  return check_launch("mla_merge_states");
}
