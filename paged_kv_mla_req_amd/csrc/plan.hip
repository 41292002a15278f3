// Split planner: cuts the (request, page) sequence of a batch into num_parts
// contiguous ranges of about equal cost, one per work-group of mla_decode.
//
// The FlashMLA backend calls get_mla_metadata once per batch step (decode
// and target-verify) and gets a [num_sm_parts, 8] tile table plus a bs+1
// split vector; only those shapes are on the page.  The rule below is this
// library's own (documented in mla_decode.h): in quarter pages, request b
// costs 4 N_b + c (c: the per-piece overhead of plan_overhead_q), part p
// covers cost positions [floor(pC/P), floor((p+1)C/P)), and a position maps
// to the nearest page boundary after dropping the first c units of its
// request.  One work-group does everything: prefix sums over requests, a
// binary search per cut for its cost position, and per-cut bookkeeping for the
// rest.  Deterministic.
#include <atomic>

#include "block_table.h"

namespace mla {

// Per-piece overhead in quarter pages: loading q and writing the result of
// rows_per_req rows (and the waits these cause), plus a constant (one page of
// the work costs 4).  On MI355X a 128-row piece costs about 3 pages
// (measured: work-group durations against their pages and pieces); the rule
// gives 3.
__host__ __device__ __forceinline__ int plan_overhead_q(int rows_per_req) {
  return 4 + (8 * rows_per_req + 127) / 128;
}

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;

// Work-group-wide exclusive prefix sum of one int per thread; *total gets
// the sum.  wave_tot: kPlanWaves ints of LDS.  Two barriers.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(inc, d, 64);
    if (lane >= d) inc += t;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    const int t = wave_tot[w];
    before += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();  // wave_tot may be reused by the next scan
  *total = all;
  return before + inc - v;
}

// First index i in [0, n) with a[i] > x (n if none).
__device__ __forceinline__ int upper_bound(const int* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] > x) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// First index i in [0, n) with a[i] >= x (n if none).
__device__ __forceinline__ int lower_bound(const int* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] >= x) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// LDS the planning work-group needs (ints).
__host__ __device__ __forceinline__ size_t plan_lds_ints(int bs, int parts) {
  return 2 * (size_t)(bs + 1) + 3 * (size_t)(parts + 1) + (size_t)(parts + 2) + kPlanWaves;
}

// The plan, computed by one work-group of 4 waves: each thread takes a
// contiguous chunk of the requests (and of the cuts) and prefix sums are
// block scans.  Each cut carries the request its cost position falls in and
// its page offset there, so the per-request piece counts and the table rows
// need no searches except where a cut sits on a request boundary.
// smem: plan_lds_ints ints.
__device__ __forceinline__ void plan_body(int* smem, const int32_t* __restrict__ seq_lens,
                                          int bs, int overhead, int parts,
                                          int32_t* __restrict__ tile_plan,
                                          int32_t* __restrict__ split_indptr) {
  // cum is dead after step 2: its space then counts each request's interior
  // cuts (extra), and after step 4 holds ubr.
  int* cum = smem;                     // [bs + 1] cost prefix (quarter pages)
  int* extra = cum;                    // [bs + 1] distinct interior cuts per request
  int* ubr = cum;                      // [bs + 1] first cut index beyond a request's start
  int* pagecum = cum + (bs + 1);       // [bs + 1] page prefix
  int* cuts = pagecum + (bs + 1);      // [parts + 1] flattened page of each cut
  int* cut_b = cuts + (parts + 1);     // [parts + 1] request of the cut's cost position
  int* cut_k = cut_b + (parts + 1);    // [parts + 1] cut page offset inside that request
  int* fcum = cut_k + (parts + 1);     // [parts + 2] prefix count of distinct interior cuts
  int* wave_tot = fcum + (parts + 2);  // [kPlanWaves]

  const int t = threadIdx.x;
  const int chunk = (bs + kPlanThreads - 1) / kPlanThreads;
  const int b_begin = min(bs, t * chunk);
  const int b_end = min(bs, b_begin + chunk);

  // 1. prefix sums of cost and pages (pages per request parked in pagecum)
  int my_cost = 0, my_pages = 0;
  for (int b = b_begin; b < b_end; ++b) {
    const int L = seq_lens[b];
    const int n = L > 0 ? (L + kPage - 1) / kPage : 0;
    pagecum[b] = n;
    my_pages += n;
    my_cost += n > 0 ? 4 * n + overhead : 0;
  }
  int C, total_pages;
  int cost_off = block_exclusive_scan(my_cost, wave_tot, &C);
  int page_off = block_exclusive_scan(my_pages, wave_tot, &total_pages);
  for (int b = b_begin; b < b_end; ++b) {
    const int n = pagecum[b];
    cum[b] = cost_off;
    pagecum[b] = page_off;
    page_off += n;
    cost_off += n > 0 ? 4 * n + overhead : 0;
  }
  if (t == 0) {
    cum[bs] = C;
    pagecum[bs] = total_pages;
  }
  __syncthreads();

  // 2. cut positions -> flattened page boundaries (nearest page boundary,
  //    the first `overhead` units of a request mapping to its page 0)
  for (int p = t; p <= parts; p += kPlanThreads) {
    int g, b = bs, k = 0;
    const int64_t x = (int64_t)p * C / parts;
    if (p == parts || x >= C) {
      g = total_pages;
    } else {
      b = upper_bound(cum, bs, (int)x) - 1;
      const int o = (int)x - cum[b];
      const int n = pagecum[b + 1] - pagecum[b];
      k = min(max(o - overhead + 2, 0) >> 2, n);
      g = pagecum[b] + k;
    }
    cuts[p] = g;
    cut_b[p] = b;
    cut_k[p] = k;
  }
  __syncthreads();
  for (int b = b_begin; b < b_end; ++b) extra[b] = 0;
  __syncthreads();

  // 3. distinct interior cuts (strictly inside a request), prefix-counted, and
  //    counted per request
  const int pchunk = (parts + 1 + kPlanThreads - 1) / kPlanThreads;
  const int p_begin = min(parts + 1, t * pchunk);
  const int p_end = min(parts + 1, p_begin + pchunk);
  auto interior = [&](int p) -> int {
    if (p < 1 || p >= parts) return 0;
    const int b = cut_b[p], k = cut_k[p];
    if (b >= bs || k <= 0 || k >= pagecum[b + 1] - pagecum[b]) return 0;
    return cuts[p] != cuts[p - 1];
  };
  int flags[4] = {0, 0, 0, 0};  // pchunk <= 3 for parts <= 512
  int my_flags = 0;
  for (int p = p_begin; p < p_end; ++p) {
    const int f = interior(p);
    if (p - p_begin < 4) flags[p - p_begin] = f;
    if (f) atomicAdd(&extra[cut_b[p]], 1);
    my_flags += f;
  }
  int n_interior;
  int fpre = block_exclusive_scan(my_flags, wave_tot, &n_interior);
  for (int p = p_begin; p < p_end; ++p) {
    fcum[p] = fpre;
    fpre += (p - p_begin < 4) ? flags[p - p_begin] : interior(p);
  }
  if (t == 0) fcum[parts + 1] = n_interior;
  __syncthreads();

  // 4. pieces per request -> split_indptr
  int my_pieces = 0;
  for (int b = b_begin; b < b_end; ++b) {
    const int np = pagecum[b + 1] > pagecum[b] ? 1 + extra[b] : 0;
    extra[b] = np;  // now the request's piece count
    my_pieces += np;
  }
  int n_pieces;
  int piece_off = block_exclusive_scan(my_pieces, wave_tot, &n_pieces);
  for (int b = b_begin; b < b_end; ++b) {
    split_indptr[b] = piece_off;
    piece_off += extra[b];
  }
  if (t == 0) split_indptr[bs] = n_pieces;
  __syncthreads();
  for (int b = b_begin; b < b_end; ++b) ubr[b] = upper_bound(cuts, parts + 1, pagecum[b]);
  __syncthreads();

  // 5. one table row per part
  for (int p = t; p < parts; p += kPlanThreads) {
    int row[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int g0 = cuts[p], g1 = cuts[p + 1];
    if (g1 > g0) {
      // request of page g0: the cut's own request unless the cut ends it
      const int cb0 = cut_b[p];
      const int b0 = (cb0 < bs && cut_k[p] < pagecum[cb0 + 1] - pagecum[cb0])
                         ? cb0
                         : upper_bound(pagecum, bs, g0) - 1;
      // request of page g1 - 1: the next cut's request unless that cut starts it
      const int b1 = (cut_b[p + 1] < bs && cut_k[p + 1] > 0)
                         ? cut_b[p + 1]
                         : upper_bound(pagecum, bs, g1 - 1) - 1;
      row[0] = b0;
      row[1] = g0 - pagecum[b0];
      row[2] = b1;
      row[3] = g1 - pagecum[b1];
      row[4] = fcum[p + 1] - fcum[ubr[b0]];
      row[5] = g1 - g0;
    }
    int4* dst = reinterpret_cast<int4*>(tile_plan + p * 8);
    dst[0] = make_int4(row[0], row[1], row[2], row[3]);
    dst[1] = make_int4(row[4], row[5], row[6], row[7]);
  }
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts inside rows of 16
// lanes, then the last lane of row 0 (and 2) added to row 1 (and 3), then the
// last lane of row 1 added to rows 2 and 3 (DPP; no LDS round trips).
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Exclusive prefix sums of N ints per thread over the work-group, with one
// barrier: wave sums go through wt (kPlanWaves * N ints of LDS, not reused
// before the next barrier).  tot[i] gets the work-group total of value i.
template <int N>
__device__ __forceinline__ void block_exclusive_sums(int (&v)[N], int* wt, int (&tot)[N]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    inc[i] = wave_inclusive_sum(v[i]);
    if (lane == 63) wt[wave * N + i] = inc[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) {
      const int t = wt[w * N + i];
      before += w < wave ? t : 0;
      all += t;
    }
    tot[i] = all;
    v[i] = before + inc[i] - v[i];
  }
}

// Exact floor / ceil of a * b / c for 0 <= a * b < 2^53 and c > 0: the quotient
// is rounded once, and a non-integer quotient is at least 1/c from the next
// integer, far more than the rounding error.
__device__ __forceinline__ int floor_mul_div(int a, int b, int c) {
  return (int)floor((double)a * (double)b / (double)c);
}
__device__ __forceinline__ int ceil_mul_div(int a, int b, int c) {
  return (int)ceil((double)a * (double)b / (double)c);
}

// LDS the small-batch planner needs (ints).
__host__ __device__ __forceinline__ size_t plan_small_lds_ints() {
  return 8 * (size_t)(kPlanThreads + 1) + 4 * kPlanWaves;
}

// The same plan as plan_body for bs <= 256 and parts <= 256 (one thread per
// request and one per part), with three barriers: each request finds the
// parts whose cost position falls inside it by division (the part range is
// [ceil(cum_b P / C), ceil(cum_{b+1} P / C))), places their cuts, counts its
// distinct interior cuts (cuts are non-decreasing) and numbers its pieces;
// the nonempty requests are listed in order, so the request before or after a
// cut that sits on a request boundary is one lookup away.
__device__ __forceinline__ void plan_small(int* smem, const int32_t* __restrict__ seq_lens,
                                           int bs, int overhead, int parts,
                                           int32_t* __restrict__ tile_plan,
                                           int32_t* __restrict__ split_indptr) {
  int* cum = smem;                               // [bs + 1] cost prefix (quarter pages)
  int* pagecum = cum + (kPlanThreads + 1);       // [bs + 1] page prefix
  int* rank = pagecum + (kPlanThreads + 1);      // [bs] index among nonempty requests
  int* ne = rank + (kPlanThreads + 1);           // [nonempty] nonempty requests in order
  int* cuts = ne + (kPlanThreads + 1);           // [parts + 1] flattened page of each cut
  int* cut_b = cuts + (kPlanThreads + 1);        // [parts + 1] request of the cut
  int* cut_k = cut_b + (kPlanThreads + 1);       // [parts + 1] page offset there
  int* first = cut_k + (kPlanThreads + 1);       // [parts] first piece index of the part
  int* wt = first + (kPlanThreads + 1);          // wave sums, 3 + 1 ints per wave

  const int t = threadIdx.x;
  const int L = t < bs ? seq_lens[t] : 0;
  const int n = L > 0 ? (L + kPage - 1) / kPage : 0;
  const int cost = n > 0 ? 4 * n + overhead : 0;
  int v[3] = {cost, n, n > 0 ? 1 : 0}, tot[3];
  block_exclusive_sums<3>(v, wt, tot);
  const int C = tot[0], total_pages = tot[1], n_ne = tot[2];
  if (t < bs) {
    cum[t] = v[0];
    pagecum[t] = v[1];
    rank[t] = v[2];
    if (n > 0) ne[v[2]] = t;
  }
  if (t == 0) {
    cum[bs] = C;
    pagecum[bs] = total_pages;
  }
  // every cut at the end, for a batch without pages (C = 0); otherwise each
  // cut p < parts is placed below by the request its cost position falls in
  if (t <= parts) cuts[t] = total_pages;
  if (t == 0 && parts == kPlanThreads) cuts[parts] = total_pages;
  __syncthreads();

  // the cuts inside request t, its distinct interior cuts and piece numbers
  int pieces = 0;
  if (t < bs && n > 0) {
    const int p_lo = ceil_mul_div(v[0], parts, C);
    const int p_hi = min(parts, ceil_mul_div(v[0] + cost, parts, C));
    int prev = -1, count = 0;
    for (int p = p_lo; p < p_hi; ++p) {
      const int o = floor_mul_div(p, C, parts) - v[0];
      const int k = min(max(o - overhead + 2, 0) >> 2, n);
      const int g = v[1] + k;
      const bool inner = p > 0 && k > 0 && k < n;
      if (inner && g != prev) ++count;
      cuts[p] = g;
      cut_b[p] = t;
      cut_k[p] = k;
      first[p] = inner ? count : 0;
      prev = g;
    }
    pieces = 1 + count;
  }
  int pv[1] = {pieces}, ptot[1];
  block_exclusive_sums<1>(pv, wt + 3 * kPlanWaves, ptot);  // also publishes the cuts
  if (t < bs) split_indptr[t] = pv[0];
  if (t == 0) split_indptr[bs] = ptot[0];

  // one table row per part
  if (t < parts) {
    int row[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int g0 = cuts[t], g1 = cuts[t + 1];
    if (g1 > g0) {
      // request of page g0: the cut's own, or the next nonempty one if the cut ends it
      const int cb0 = cut_b[t];
      const int b0 = cut_k[t] < pagecum[cb0 + 1] - pagecum[cb0] ? cb0 : ne[rank[cb0] + 1];
      // request of page g1 - 1: the next cut's own, or the nonempty one before
      // it if that cut starts its request (or the last one for the final cut)
      int b1;
      if (t + 1 == parts) {
        b1 = ne[n_ne - 1];
      } else {
        const int cb1 = cut_b[t + 1];
        b1 = cut_k[t + 1] > 0 ? cb1 : ne[rank[cb1] - 1];
      }
      row[0] = b0;
      row[1] = g0 - pagecum[b0];
      row[2] = b1;
      row[3] = g1 - pagecum[b1];
      row[4] = first[t];
      row[5] = g1 - g0;
    }
    int4* dst = reinterpret_cast<int4*>(tile_plan + t * 8);
    dst[0] = make_int4(row[0], row[1], row[2], row[3]);
    dst[1] = make_int4(row[4], row[5], row[6], row[7]);
  }
}

// The planning work-group: the small-batch form when it applies.
__device__ __forceinline__ void plan(int* smem, const int32_t* __restrict__ seq_lens, int bs,
                                     int overhead, int parts, int32_t* __restrict__ tile_plan,
                                     int32_t* __restrict__ split_indptr) {
  if (bs <= kPlanThreads && parts <= kPlanThreads)
    plan_small(smem, seq_lens, bs, overhead, parts, tile_plan, split_indptr);
  else
    plan_body(smem, seq_lens, bs, overhead, parts, tile_plan, split_indptr);
}

__global__ void __launch_bounds__(kPlanThreads)
plan_splits_kernel(const int32_t* __restrict__ seq_lens, int bs, int overhead, int parts,
                   int32_t* __restrict__ tile_plan, int32_t* __restrict__ split_indptr) {
  extern __shared__ int smem[];
  plan(smem, seq_lens, bs, overhead, parts, tile_plan, split_indptr);
}

// Block table and plan in one launch (init_forward_metadata computes both
// for a batch step): work-group 0 plans, the others fill the table, 256 cells
// of one request each, while the plan's dependent steps run.
__global__ void __launch_bounds__(kPlanThreads)
table_and_plan_kernel(const int32_t* __restrict__ req_to_token, int32_t r2t_rows,
                      int64_t r2t_row_stride, const int32_t* __restrict__ req_pool_indices,
                      const int32_t* __restrict__ seq_lens, int32_t* __restrict__ block_table,
                      int32_t bt_row_stride, int32_t pad_value, int bt_blocks_per_row, int bs,
                      int overhead, int parts, int32_t* __restrict__ tile_plan,
                      int32_t* __restrict__ split_indptr) {
  extern __shared__ int smem[];
  if (blockIdx.x == 0) {
    plan(smem, seq_lens, bs, overhead, parts, tile_plan, split_indptr);
    return;
  }
  const int w = blockIdx.x - 1;
  const int b = w / bt_blocks_per_row;
  const int p = (w - b * bt_blocks_per_row) * kPlanThreads + threadIdx.x;
  if (p < bt_row_stride)
    block_table_cell(b, p, req_to_token, r2t_rows, r2t_row_stride, req_pool_indices, seq_lens,
                     block_table, bt_row_stride, pad_value);
}

}  // namespace mla

namespace mla {

mla_status check_plan_args(const char* who, const int32_t* seq_lens, int32_t bs,
                           int32_t rows_per_req, int32_t num_parts, int32_t kv_dtype,
                           const int32_t* tile_plan, const int32_t* split_indptr) {
  const std::string w(who);
  if (!seq_lens || !tile_plan || !split_indptr)
    return fail(MLA_ERR_INVALID_ARGUMENT, w + ": null pointer");
  if (bs <= 0 || num_parts <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, w + ": bs and num_parts must be positive");
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_INVALID_ARGUMENT, w + ": unknown kv_dtype");
  if (rows_per_req < 1 || rows_per_req > MLA_MAX_ROWS_PER_REQ)
    return fail(MLA_ERR_UNSUPPORTED, w + ": rows_per_req must be in 1..512");
  if (reinterpret_cast<uintptr_t>(tile_plan) & 15u)
    return fail(MLA_ERR_UNSUPPORTED, w + ": tile_plan must be 16-byte aligned");
  if (bs > MLA_MAX_BATCH)
    return fail(MLA_ERR_CAPACITY, w + ": bs above " + std::to_string(MLA_MAX_BATCH));
  if (num_parts > MLA_MAX_PARTS)
    return fail(MLA_ERR_CAPACITY, w + ": num_parts above " + std::to_string(MLA_MAX_PARTS));
  int cus = mla_device_num_cus();
  if (cus > 0 && num_parts > cus)
    return fail(MLA_ERR_CAPACITY, w + ": num_parts " + std::to_string(num_parts) +
                                      " exceeds the device's " + std::to_string(cus) + " CUs");
  return MLA_OK;
}

// LDS ints of the planning work-group for a batch.
inline size_t plan_lds(int bs, int parts) {
  return (bs <= kPlanThreads && parts <= kPlanThreads) ? plan_small_lds_ints()
                                                       : plan_lds_ints(bs, parts);
}

// Raises the dynamic-LDS limit of a planning kernel once per device (the
// attribute is set for the current device).  `done` holds one flag per device
// ordinal; calls from several host threads may both set it, which is harmless.
constexpr int kMaxDevices = 64;
template <typename K>
mla_status allow_plan_lds(K kernel, std::atomic<bool> (&done)[kMaxDevices], const char* who) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess)
    return fail(MLA_ERR_DEVICE, std::string(who) + ": no current device");
  if (dev < 0 || dev >= kMaxDevices || !done[dev].load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024) != hipSuccess)
      return fail(MLA_ERR_DEVICE, std::string(who) + ": cannot raise the LDS limit");
    if (dev >= 0 && dev < kMaxDevices) done[dev].store(true, std::memory_order_release);
  }
  return MLA_OK;
}

}  // namespace mla

extern "C" mla_status mla_plan_splits(const int32_t* seq_lens, int32_t bs, int32_t rows_per_req,
                                      int32_t num_parts, int32_t kv_dtype, int32_t* tile_plan,
                                      int32_t* split_indptr, hipStream_t stream) {
  using namespace mla;
  const mla_status st = check_plan_args("mla_plan_splits", seq_lens, bs, rows_per_req, num_parts,
                                        kv_dtype, tile_plan, split_indptr);
  if (st != MLA_OK) return st;
  const int overhead = plan_overhead_q(rows_per_req);
  const size_t lds = sizeof(int) * plan_lds(bs, num_parts);
  static std::atomic<bool> lds_raised[kMaxDevices];
  const mla_status la = allow_plan_lds(plan_splits_kernel, lds_raised, "mla_plan_splits");
  if (la != MLA_OK) return la;
  trace("mla_plan_splits: bs %d rows %d parts %d lds %zu stream %p", bs, rows_per_req, num_parts,
        lds, (void*)stream);
  hipLaunchKernelGGL(plan_splits_kernel, dim3(1), dim3(kPlanThreads), lds, stream, seq_lens, bs,
                     overhead, num_parts, tile_plan, split_indptr);
  return check_launch("mla_plan_splits");
}

extern "C" mla_status mla_build_table_and_plan(
    const int32_t* req_to_token, int32_t r2t_rows, int64_t r2t_row_stride,
    const int32_t* req_pool_indices, const int32_t* seq_lens, int32_t bs, int32_t page_size,
    int32_t* block_table, int32_t bt_row_stride, int32_t pad_value, int32_t max_seq_len_hint,
    int32_t rows_per_req, int32_t num_parts, int32_t kv_dtype, int32_t* tile_plan,
    int32_t* split_indptr, hipStream_t stream) {
  using namespace mla;
  const char* who = "mla_build_table_and_plan";
  mla_status st = check_block_table_args(who, req_to_token, r2t_rows, r2t_row_stride,
                                         req_pool_indices, seq_lens, bs, page_size, block_table,
                                         bt_row_stride, max_seq_len_hint);
  if (st != MLA_OK) return st;
  st = check_plan_args(who, seq_lens, bs, rows_per_req, num_parts, kv_dtype, tile_plan,
                       split_indptr);
  if (st != MLA_OK) return st;
  const int per_row = (bt_row_stride + kPlanThreads - 1) / kPlanThreads;
  const int64_t blocks = 1 + (int64_t)bs * per_row;
  if (blocks > 0x7fffffff) return fail(MLA_ERR_UNSUPPORTED, std::string(who) + ": table too large");
  const size_t lds = sizeof(int) * plan_lds(bs, num_parts);
  static std::atomic<bool> lds_raised[kMaxDevices];
  st = allow_plan_lds(table_and_plan_kernel, lds_raised, who);
  if (st != MLA_OK) return st;
  trace("%s: bs %d width %d rows %d parts %d grid %lld lds %zu stream %p", who, bs,
        bt_row_stride, rows_per_req, num_parts, (long long)blocks, lds, (void*)stream);
  hipLaunchKernelGGL(table_and_plan_kernel, dim3((unsigned)blocks), dim3(kPlanThreads), lds,
                     stream, req_to_token, r2t_rows, r2t_row_stride, req_pool_indices, seq_lens,
                     block_table, bt_row_stride, pad_value, per_row, bs,
                     plan_overhead_q(rows_per_req), num_parts, tile_plan, split_indptr);
#ifdef MLA_DEBUG
  st = check_launch(who);
  if (st != MLA_OK) return st;
  return debug_check_page_aligned(who, req_to_token, r2t_rows, r2t_row_stride, req_pool_indices,
                                  seq_lens, bs, block_table, bt_row_stride, stream);
#else
  return check_launch(who);
#endif
}

// ---------------------------------------------------------------------------
// Fixed-tile planner (the FlashInfer backend page's deterministic mode: with
// enable_deterministic the decode KV is split into tiles of
// decode_split_tile_size = 2048 tokens and graph-mode KV splitting is off).
// Request b is cut at the multiples of tile_pages pages of its own sequence,
// so its pieces -- and so the arithmetic of its result -- do not depend on
// the rest of the batch.  Piece k of request b is part split_indptr[b] + k.
// One work-group: two passes of block scans over chunks of 256 requests (the
// first only counts), then the rows past the last piece are cleared.
namespace mla {

__device__ __forceinline__ int fixed_pieces(int32_t L, int tile_pages, int cap) {
  const int np = L > 0 ? (L >> 6) + ((L & (kPage - 1)) != 0) : 0;
  return min(np / tile_pages + (np % tile_pages != 0), cap);
}

__global__ __launch_bounds__(kPlanThreads) void plan_fixed_kernel(
    const int32_t* __restrict__ seq_lens, int32_t bs, int32_t tile_pages, int32_t max_parts,
    int32_t* __restrict__ tile_plan, int32_t* __restrict__ split_indptr) {
  __shared__ int wave_tot[kPlanWaves];
  // A request's count is capped at max_parts + 1: the sum of at most 16384
  // capped counts fits an int, and any capped request already overflows.
  const int cap = max_parts + 1;
  int total = 0;
  for (int c0 = 0; c0 < bs; c0 += kPlanThreads) {
    const int b = c0 + (int)threadIdx.x;
    const int n = b < bs ? fixed_pieces(seq_lens[b], tile_pages, cap) : 0;
    int chunk_total;
    block_exclusive_scan(n, wave_tot, &chunk_total);
    total = min(total + chunk_total, cap);
  }
  const bool fits = total <= max_parts;
  int base = 0;
  for (int c0 = 0; fits && c0 < bs; c0 += kPlanThreads) {
    const int b = c0 + (int)threadIdx.x;
    const int n = b < bs ? fixed_pieces(seq_lens[b], tile_pages, cap) : 0;
    int chunk_total;
    const int before = base + block_exclusive_scan(n, wave_tot, &chunk_total);
    if (b < bs) {
      split_indptr[b] = before;
      const int np = seq_lens[b] > 0 ? (seq_lens[b] >> 6) + ((seq_lens[b] & (kPage - 1)) != 0)
                                     : 0;
      for (int k = 0; k < n; ++k) {
        const int pg0 = k * tile_pages, pg1 = min(pg0 + tile_pages, np);
        int32_t* row = tile_plan + (int64_t)(before + k) * 8;
        *reinterpret_cast<int4*>(row) = make_int4(b, pg0, b, pg1);
        *reinterpret_cast<int4*>(row + 4) = make_int4(k, pg1 - pg0, 0, 0);
      }
    }
    base += chunk_total;
  }
  // Without room, nothing is planned: split_indptr and every row are 0.
  const int used = fits ? total : 0;
  if (!fits)
    for (int b = (int)threadIdx.x; b < bs; b += kPlanThreads) split_indptr[b] = 0;
  if (threadIdx.x == 0) split_indptr[bs] = used;
  for (int64_t i = (int64_t)used * 8 + threadIdx.x; i < (int64_t)max_parts * 8; i += kPlanThreads)
    tile_plan[i] = 0;
}

// Packed fixed-tile plan: the tiles of plan_fixed_kernel (the same pieces and
// split_indptr), in request order, cut into `parts` contiguous runs of about
// equal cost.  In quarter pages a tile of n pages costs 4 n + overhead; with
// Q_t the cost before tile t and x_p = floor(p C / parts), cut p is the tile
// boundary whose Q_t is nearest x_p (the lower one on a tie).  Each thread
// finds its cuts by one binary search over the requests' cost prefix and a
// division inside the request (its tiles but the last cost the same); the
// row then needs the requests of its first and last tile.
// LDS: 2 (bs + 1) + parts + 1 + kPlanWaves ints.
__global__ __launch_bounds__(kPlanThreads) void plan_fixed_packed_kernel(
    const int32_t* __restrict__ seq_lens, int32_t bs, int32_t tile_pages, int32_t overhead,
    int32_t parts, int32_t* __restrict__ tile_plan, int32_t* __restrict__ split_indptr) {
  extern __shared__ int smem[];
  int* tpre = smem;                    // [bs + 1] tiles before request b
  int* cpre = tpre + (bs + 1);         // [bs + 1] cost before request b
  int* cuts = cpre + (bs + 1);         // [parts + 1] first tile of part p
  int* wave_tot = cuts + (parts + 1);  // [kPlanWaves]
  const int t = threadIdx.x, T = tile_pages;
  const int chunk = (bs + kPlanThreads - 1) / kPlanThreads;
  const int b_begin = min(bs, t * chunk);
  const int b_end = min(bs, b_begin + chunk);

  // 1. tiles and cost per request, prefix sums; split_indptr = tile prefix
  int my_tiles = 0, my_cost = 0;
  for (int b = b_begin; b < b_end; ++b) {
    const int32_t L = seq_lens[b];
    const int np = L > 0 ? (L >> 6) + ((L & (kPage - 1)) != 0) : 0;
    const int n = np / T + (np % T != 0);
    tpre[b] = n;
    cpre[b] = 4 * np + overhead * n;
    my_tiles += n;
    my_cost += 4 * np + overhead * n;
  }
  int NT, C;
  int toff = block_exclusive_scan(my_tiles, wave_tot, &NT);
  int coff = block_exclusive_scan(my_cost, wave_tot, &C);
  for (int b = b_begin; b < b_end; ++b) {
    const int n = tpre[b], c = cpre[b];
    tpre[b] = toff;
    cpre[b] = coff;
    split_indptr[b] = toff;
    toff += n;
    coff += c;
  }
  if (t == 0) {
    tpre[bs] = NT;
    cpre[bs] = C;
    split_indptr[bs] = NT;
  }
  __syncthreads();

  // 2. cuts: the tile boundary nearest each cost position
  const int w = 4 * T + overhead;  // cost of every tile of a request but its last
  for (int p = t; p <= parts; p += kPlanThreads) {
    int cut = NT;
    const int64_t x64 = (int64_t)p * C / parts;
    if (p == 0) {
      cut = 0;
    } else if (p < parts && x64 < C) {
      const int x = (int)x64;
      const int b = upper_bound(cpre, bs, x) - 1;  // cpre[b] <= x < cpre[b + 1]
      const int o = x - cpre[b];
      const int n = tpre[b + 1] - tpre[b];
      const int k0 = min(o / w, n - 1);
      const int q0 = k0 * w;
      const int q1 = k0 + 1 < n ? (k0 + 1) * w : cpre[b + 1] - cpre[b];
      cut = tpre[b] + (o - q0 <= q1 - o ? k0 : k0 + 1);
    }
    cuts[p] = cut;
  }
  __syncthreads();

  // 3. one row per part
  auto pages_before = [&](int b) { return (cpre[b] - overhead * tpre[b]) >> 2; };
  for (int p = t; p < parts; p += kPlanThreads) {
    int row[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int t0 = cuts[p], t1 = cuts[p + 1];
    if (t1 > t0) {
      const int b0 = upper_bound(tpre, bs, t0) - 1;
      const int k0 = t0 - tpre[b0];
      const int b1 = upper_bound(tpre, bs, t1 - 1) - 1;
      const int k1 = t1 - 1 - tpre[b1];
      const int np1 = pages_before(b1 + 1) - pages_before(b1);
      const int pg1 = min((k1 + 1) * T, np1);
      row[0] = b0;
      row[1] = k0 * T;
      row[2] = b1;
      row[3] = pg1;
      row[4] = k0;
      row[5] = (pages_before(b1) + pg1) - (pages_before(b0) + k0 * T);
      row[6] = T;
    }
    int4* dst = reinterpret_cast<int4*>(tile_plan + p * 8);
    dst[0] = make_int4(row[0], row[1], row[2], row[3]);
    dst[1] = make_int4(row[4], row[5], row[6], row[7]);
  }
}

// ceil(ceil(max_seq_len / 64) / tile_pages) pieces per request, times bs;
// -1 for bad arguments, INT32_MAX when the count does not fit.
int64_t fixed_parts_bound(int32_t bs, int32_t max_seq_len, int32_t tile_pages) {
  if (bs < 0 || max_seq_len < 0 || tile_pages <= 0) return -1;
  const int64_t np = ((int64_t)max_seq_len + kPage - 1) / kPage;
  return (int64_t)bs * ((np + tile_pages - 1) / tile_pages);
}

}  // namespace mla

extern "C" int32_t mla_fixed_split_parts_bound(int32_t bs, int32_t max_seq_len,
                                               int32_t tile_pages) {
  const int64_t v = mla::fixed_parts_bound(bs, max_seq_len, tile_pages);
  return v > INT32_MAX ? INT32_MAX : (int32_t)v;
}

extern "C" mla_status mla_plan_fixed_splits(const int32_t* seq_lens, int32_t bs,
                                            int32_t tile_pages, int32_t max_parts,
                                            int32_t max_seq_len_hint, int32_t* tile_plan,
                                            int32_t* split_indptr, hipStream_t stream) {
  using namespace mla;
  const std::string w("mla_plan_fixed_splits");
  if (!seq_lens || !tile_plan || !split_indptr)
    return fail(MLA_ERR_INVALID_ARGUMENT, w + ": null pointer");
  if (bs <= 0 || tile_pages <= 0 || max_parts <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, w + ": bs, tile_pages and max_parts must be positive");
  if (bs > MLA_MAX_BATCH)
    return fail(MLA_ERR_CAPACITY, w + ": bs above " + std::to_string(MLA_MAX_BATCH));
  if (max_parts > MLA_MAX_DECODE_PARTS)
    return fail(MLA_ERR_CAPACITY, w + ": max_parts above " + std::to_string(MLA_MAX_DECODE_PARTS));
  if (reinterpret_cast<uintptr_t>(tile_plan) & 15u)
    return fail(MLA_ERR_UNSUPPORTED, w + ": tile_plan must be 16-byte aligned");
  if (max_seq_len_hint >= 0 && fixed_parts_bound(bs, max_seq_len_hint, tile_pages) > max_parts)
    return fail(MLA_ERR_CAPACITY, w + ": " + std::to_string(bs) + " requests of up to " +
                                      std::to_string(max_seq_len_hint) +
                                      " tokens may need more than max_parts pieces");
  trace("%s: bs %d tile_pages %d max_parts %d stream %p", w.c_str(), bs, tile_pages, max_parts,
        (void*)stream);
  hipLaunchKernelGGL(plan_fixed_kernel, dim3(1), dim3(kPlanThreads), 0, stream, seq_lens, bs,
                     tile_pages, max_parts, tile_plan, split_indptr);
  return check_launch(w.c_str());
}

extern "C" mla_status mla_plan_fixed_packed(const int32_t* seq_lens, int32_t bs,
                                            int32_t tile_pages, int32_t rows_per_req,
                                            int32_t num_parts, int32_t* tile_plan,
                                            int32_t* split_indptr, hipStream_t stream) {
  using namespace mla;
  const char* who = "mla_plan_fixed_packed";
  const std::string w(who);
  if (tile_pages <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, w + ": tile_pages must be positive");
  const mla_status st = check_plan_args(who, seq_lens, bs, rows_per_req, num_parts, MLA_KV_BF16,
                                        tile_plan, split_indptr);
  if (st != MLA_OK) return st;
  const size_t lds = sizeof(int) * (2 * (size_t)(bs + 1) + (size_t)num_parts + 1 + kPlanWaves);
  static std::atomic<bool> lds_raised[kMaxDevices];
  const mla_status la = allow_plan_lds(plan_fixed_packed_kernel, lds_raised, who);
  if (la != MLA_OK) return la;
  trace("%s: bs %d tile_pages %d rows %d parts %d lds %zu stream %p", who, bs, tile_pages,
        rows_per_req, num_parts, lds, (void*)stream);
  hipLaunchKernelGGL(plan_fixed_packed_kernel, dim3(1), dim3(kPlanThreads), lds, stream, seq_lens,
                     bs, tile_pages, plan_overhead_q(rows_per_req), num_parts, tile_plan,
                     split_indptr);
  return check_launch(who);
}
