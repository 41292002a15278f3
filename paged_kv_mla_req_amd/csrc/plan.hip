// Split planner: cuts the (request, page) sequence of a batch into num_parts
// contiguous ranges of about equal cost, one per work-group of mla_decode.
//
// The FlashMLA backend calls get_mla_metadata once per batch step (decode
// and target-verify) and gets a [num_sm_parts, 8] tile table plus a bs+1
// split vector; only those shapes are on the page.  The rule below is this
// library's own (documented in mla_decode.h): request b costs N_b + c page
// units, part p covers cost positions [floor(pC/P), floor((p+1)C/P)), and a
// position maps to a page boundary by dropping the first c units of each
// request.  Everything runs in one work-group: prefix sums over requests,
// one thread per cut, binary searches for the rest.  Deterministic.
#include "common.h"

namespace mla {

constexpr int kPlanThreads = 1024;

// Exclusive prefix sum of one int per thread over the whole block; returns
// this thread's prefix and writes the block total to *total.
__device__ int block_exclusive_scan(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int t = __shfl_up(inc, d, 64);
    if (lane >= d) inc += t;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      int t = wave_tot[w];
      wave_tot[w] = run;
      run += t;
    }
    *total = run;
  }
  __syncthreads();
  int res = inc - v + wave_tot[wave];
  __syncthreads();
  return res;
}

// First index i in [0, n) with a[i] > x (n if none).
__device__ __forceinline__ int upper_bound(const int* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (a[mid] > x) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// First index i in [0, n) with a[i] >= x (n if none).
__device__ __forceinline__ int lower_bound(const int* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (a[mid] >= x) hi = mid; else lo = mid + 1;
  }
  return lo;
}

__global__ void __launch_bounds__(kPlanThreads)
plan_splits_kernel(const int32_t* __restrict__ seq_lens, int bs, int overhead, int parts,
                   int32_t* __restrict__ tile_plan, int32_t* __restrict__ split_indptr) {
  extern __shared__ int smem[];
  int* cum = smem;                    // [bs + 1] cost prefix
  int* pagecum = cum + (bs + 1);      // [bs + 1] page prefix
  int* cuts = pagecum + (bs + 1);     // [parts + 1] flattened page of each cut
  int* fcum = cuts + (parts + 1);     // [parts + 2] prefix count of distinct interior cuts
  int* wave_tot = fcum + (parts + 2); // [16]
  int* totals = wave_tot + 16;        // [4]

  const int t = threadIdx.x;
  const int chunk = (bs + kPlanThreads - 1) / kPlanThreads;
  const int b_begin = min(bs, t * chunk);
  const int b_end = min(bs, b_begin + chunk);

  // 1. prefix sums of cost and pages
  int my_cost = 0, my_pages = 0;
  for (int b = b_begin; b < b_end; ++b) {
    int L = seq_lens[b];
    int n = L > 0 ? (L + kPage - 1) / kPage : 0;
    my_pages += n;
    my_cost += n > 0 ? n + overhead : 0;
  }
  int cost_off = block_exclusive_scan(my_cost, wave_tot, &totals[0]);
  int page_off = block_exclusive_scan(my_pages, wave_tot, &totals[1]);
  for (int b = b_begin; b < b_end; ++b) {
    int L = seq_lens[b];
    int n = L > 0 ? (L + kPage - 1) / kPage : 0;
    cum[b] = cost_off;
    pagecum[b] = page_off;
    page_off += n;
    cost_off += n > 0 ? n + overhead : 0;
  }
  if (t == 0) {
    cum[bs] = totals[0];
    pagecum[bs] = totals[1];
  }
  __syncthreads();
  const int C = cum[bs];
  const int total_pages = pagecum[bs];

  // 2. cut positions -> flattened page boundaries
  if (t <= parts) {
    int g;
    const int64_t x = (int64_t)t * C / parts;
    if (t == parts || x >= C) {
      g = total_pages;
    } else {
      int b = upper_bound(cum, bs, (int)x) - 1;
      int o = (int)x - cum[b];
      int n = pagecum[b + 1] - pagecum[b];
      g = pagecum[b] + min(max(o - overhead, 0), n);
    }
    cuts[t] = g;
  }
  __syncthreads();

  // 3. distinct interior cuts (strictly inside a request), prefix-counted
  int flag = 0;
  if (t >= 1 && t < parts) {
    int g = cuts[t];
    if (g > 0 && g < total_pages && g != cuts[t - 1]) {
      int b = upper_bound(pagecum, bs, g) - 1;
      flag = (g - pagecum[b]) > 0;
    }
  }
  int fpre = block_exclusive_scan(t <= parts ? flag : 0, wave_tot, &totals[2]);
  if (t <= parts) fcum[t] = fpre;
  if (t == 0) fcum[parts + 1] = totals[2];
  __syncthreads();

  // 4. pieces per request -> split_indptr
  int my_pieces = 0;
  for (int b = b_begin; b < b_end; ++b) {
    int lo = pagecum[b], hi = pagecum[b + 1];
    if (hi == lo) continue;
    int i_lo = upper_bound(cuts, parts + 1, lo);
    int i_hi = lower_bound(cuts, parts + 1, hi);
    my_pieces += 1 + (i_hi > i_lo ? fcum[i_hi] - fcum[i_lo] : 0);
  }
  int piece_off = block_exclusive_scan(my_pieces, wave_tot, &totals[3]);
  for (int b = b_begin; b < b_end; ++b) {
    split_indptr[b] = piece_off;
    int lo = pagecum[b], hi = pagecum[b + 1];
    if (hi == lo) continue;
    int i_lo = upper_bound(cuts, parts + 1, lo);
    int i_hi = lower_bound(cuts, parts + 1, hi);
    piece_off += 1 + (i_hi > i_lo ? fcum[i_hi] - fcum[i_lo] : 0);
  }
  if (t == 0) split_indptr[bs] = totals[3];

  // 5. one table row per part
  if (t < parts) {
    int row[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int g0 = cuts[t], g1 = cuts[t + 1];
    if (g1 > g0) {
      int b0 = upper_bound(pagecum, bs, g0) - 1;
      int b1 = upper_bound(pagecum, bs, g1 - 1) - 1;
      row[0] = b0;
      row[1] = g0 - pagecum[b0];
      row[2] = b1;
      row[3] = g1 - pagecum[b1];
      row[4] = fcum[upper_bound(cuts, parts + 1, g0)] - fcum[upper_bound(cuts, parts + 1, pagecum[b0])];
      row[5] = g1 - g0;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) tile_plan[t * 8 + k] = row[k];
  }
}

}  // namespace mla

extern "C" mla_status mla_plan_splits(const int32_t* seq_lens, int32_t bs, int32_t rows_per_req,
                                      int32_t num_parts, int32_t kv_dtype, int32_t* tile_plan,
                                      int32_t* split_indptr, hipStream_t stream) {
  using namespace mla;
  if (!seq_lens || !tile_plan || !split_indptr)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_plan_splits: null pointer");
  if (bs <= 0 || num_parts <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_plan_splits: bs and num_parts must be positive");
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_plan_splits: unknown kv_dtype");
  if (rows_per_req < 1 || rows_per_req > MLA_MAX_ROWS_PER_REQ)
    return fail(MLA_ERR_UNSUPPORTED, "mla_plan_splits: rows_per_req must be in 1..512");
  if (bs > MLA_MAX_BATCH)
    return fail(MLA_ERR_CAPACITY, "mla_plan_splits: bs above " + std::to_string(MLA_MAX_BATCH));
  if (num_parts > MLA_MAX_PARTS)
    return fail(MLA_ERR_CAPACITY, "mla_plan_splits: num_parts above " + std::to_string(MLA_MAX_PARTS));
  int cus = mla_device_num_cus();
  if (cus > 0 && num_parts > cus)
    return fail(MLA_ERR_CAPACITY, "mla_plan_splits: num_parts " + std::to_string(num_parts) +
                                      " exceeds the device's " + std::to_string(cus) + " CUs");
  const int overhead = 1 + rows_per_req / 64;
  const size_t lds = sizeof(int) * (2 * (size_t)(bs + 1) + (size_t)(num_parts + 1) +
                                    (size_t)(num_parts + 2) + 16 + 4);
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)plan_splits_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
      return fail(MLA_ERR_DEVICE, "mla_plan_splits: cannot raise the LDS limit");
    attr_set = true;
  }
  hipLaunchKernelGGL(plan_splits_kernel, dim3(1), dim3(kPlanThreads), lds, stream, seq_lens, bs,
                     overhead, num_parts, tile_plan, split_indptr);
  return check_launch("mla_plan_splits");
}
