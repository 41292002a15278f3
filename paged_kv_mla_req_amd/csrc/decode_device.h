// Device helpers shared by the decode kernels (decode.hip: bf16 cache and
// e4m3 cache with a bf16 query; decode_q8.hip: e4m3 cache with an e4m3
// query): sizes and layouts, the page loads, the inline-assembly MFMA chains
// and their operand reads, the softmax helpers and the output epilogue.  The
// layouts and chains are described where they are defined; the kernels'
// own files describe how they use them.
#pragma once

#include <cmath>
#include <utility>

#include <hip/hip_ext.h>

#include "common.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;     // 128
constexpr int kRowBytes = kD * 2;                        // 1152 bytes per bf16 latent row
constexpr int kChunks = kRowBytes / 16;                  // 72 16-byte chunks per row
constexpr int kPageBytes = kPage * kRowBytes;            // 73728
constexpr int kPageBytesF8 = kPage * kD;                 // 36864: one e4m3 page
constexpr int kLoadsPerWaveF8 = kPageBytesF8 / 1024 / kWaves;  // 9
constexpr int kLoadsPerPage = kPageBytes / 1024;         // 72 wave-wide 1 KiB loads
constexpr int kLoadsPerWave = kLoadsPerPage / kWaves;    // 18
constexpr int kKSteps = kD / 16;                         // 36 MFMA k-steps for S
constexpr int kVTiles = kDv / 32;                        // 16 output tiles of 32 columns
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr int kXcds = 8;      // accelerator dies, each with its own L2

// Work-groups go to the dies round robin (work-group i to die i % 8).
// Neighbouring parts mostly hold pieces of the same request, which load the
// same query rows: part_of_block gives each die a contiguous run of parts, so
// those loads hit the die's L2 after the first.  A bijection of [0, parts).
__device__ __forceinline__ int part_of_block(int i, int parts) {
  const int x = i % kXcds, j = i / kXcds;
  const int per = parts / kXcds, extra = parts % kXcds;
  return x * per + min(x, extra) + j;
}
// The page loop issues the next page's loads one per block of four MFMAs of
// the first score tile (e4m3: all 9; bf16: 9 of 18), the rest of bf16 one
// every third slot early in the second tile's chain.
static_assert(kLoadsPerWave == 18 && kLoadsPerWaveF8 == 9 && kKSteps / 4 == 9,
              "load spreading assumes 18 / 9 loads and 9 score blocks");

// Scalar arguments of the decode kernel (pointers are kernel arguments of
// their own, marked __restrict__, so the compiler may read the small index
// arrays through the scalar cache).
struct DecodeParams {
  int64_t num_pages;
  int32_t partial_slots;      // capacity of partial_o / partial_lse
  int32_t bt_stride;
  int32_t bs;
  int32_t q_len;
  int32_t heads;
  int32_t rows;               // R = q_len * heads
  int32_t causal;
  float scale_log2;           // softmax_scale * log2(e)
};

// Buffer resource for one page: base = the page, range = its first `rows`
// latent rows.  Loads past the range return zeros, so the slots of a last
// page beyond the request's length arrive in LDS as zeros whatever the pool
// holds there (a masked key then contributes 0 * 0, never 0 * NaN).
template <int RowBytes>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t* page, int rows) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(page), (short)0,
                                           rows * RowBytes, 0x00020000);
}

// Cache policy of the page loads: non-temporal (the nt bit).  Every latent
// page is read once per launch, so the loads are marked as streaming and do
// not push the reused lines -- a request's query rows, which the pieces on one
// die share, and the partial states -- out of the die's L2.  Measured on the
// DeepSeek-V3-shaped batch, same box, alternating builds: decode 93.2 -> 87.1 us
// and 96.6 -> 90.5 us; fp8 cache 161.2 -> 160.1 us.  (Non-temporal stores of
// the outputs made the decode 1.3% faster and the merge, which reads them, as
// much slower, so the stores keep the default policy.)
constexpr int kStreamLoad = 2;

// Issue this wave's share of the direct-to-LDS loads of one page.  Load j
// (wave w issues j = w + 4k, k = 0..17) fills LDS bytes [1024 j, 1024 j + 1024):
// column block j / 8 = k / 2, keys 8 (j % 8) .. +7 with j % 8 = w + 4 (k % 2).
// Lane i writes chunk slot i % 8 of key 8 (j % 8) + i / 8, reading global
// chunk (i % 8) ^ swz(key) of that block.  voff[k % 2] holds the lane's
// source offset for its key group; the column block is the immediate offset.
// The whole offset is in the VGPR so that the range check covers it.
// The instruction's immediate offset moves the LDS destination as well as
// the source (LDS address = M0 + offset + 16 * lane), so M0 is set that much
// lower than the destination.
template <int K>
__device__ __forceinline__ void issue_one_load(__amdgpu_buffer_rsrc_t rsrc, uint8_t* buf,
                                               int wave, uint32_t voff0, uint32_t voff1) {
  const int j = wave + kWaves * K;
  constexpr int imm = (K >> 1) * 128;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, buf + j * 1024 - imm), 16,
                                           (K & 1) ? voff1 : voff0, 0, imm, kStreamLoad);
}

template <int... K>
__device__ __forceinline__ void issue_loads(std::integer_sequence<int, K...>,
                                            __amdgpu_buffer_rsrc_t rsrc, uint8_t* buf, int wave,
                                            uint32_t voff0, uint32_t voff1) {
  (issue_one_load<K>(rsrc, buf, wave, voff0, voff1), ...);
}

__device__ __forceinline__ void issue_page_loads(__amdgpu_buffer_rsrc_t rsrc, uint8_t* buf,
                                                 int wave, uint32_t voff0, uint32_t voff1) {
  issue_loads(std::make_integer_sequence<int, kLoadsPerWave>{}, rsrc, buf, wave, voff0, voff1);
}

// The lane's index in its wave, from the execution mask (two VALU
// instructions), so that no register has to carry the work-item id through
// the kernel.
__device__ __forceinline__ uint32_t lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// e4m3 page: a plain copy into a 36 KiB staging buffer.  Load k of wave w
// fills staging bytes [1024 j, 1024 j + 1024) with j = w + 4k from the same
// page offsets; voff = 1024 w + 16 lane.
template <int... K>
__device__ __forceinline__ void issue_loads_f8(std::integer_sequence<int, K...>,
                                               __amdgpu_buffer_rsrc_t rsrc, uint8_t* stage,
                                               int wave, uint32_t voff) {
  (__builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc,
                                            LDS_PTR(void, stage + 1024 * (wave + kWaves * K)),
                                            16, voff + 4096 * K, 0, 0, kStreamLoad),
   ...);
}

template <int K>
__device__ __forceinline__ void issue_one_load_f8(__amdgpu_buffer_rsrc_t rsrc, uint8_t* stage,
                                                  int wave, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, stage + 1024 * (wave + kWaves * K)),
                                           16, voff + 4096 * K, 0, 0, kStreamLoad);
}

// Swizzle of the 16-byte chunks of key k in a column block (see the top).
__device__ __forceinline__ int chunk_swz(int k) {
  return 4 * ((k >> 1) & 1) + 2 * ((k >> 2) & 1) + ((k >> 4) & 1);
}

// Staged e4m3 page -> bf16 compute page.  Thread t converts key t / 4,
// 16-byte staging chunks j = t % 4 + 4 m (columns 16 j .. 16 j + 15) for
// m = 0..8, i.e. the chunk pair 2 (t % 4), 2 (t % 4) + 1 of column block m.
// The conversion is exact.  All addresses are a per-thread base plus a
// constant, so nothing is kept per m.
__device__ __forceinline__ void convert_f8_page(const uint8_t* stage, uint8_t* buf, int wave) {
  const int tid = wave * 64 + (int)lane_id();
  const int key = tid >> 2;
  const int c0 = 2 * (tid & 3);
  const int slot0 = c0 ^ chunk_swz(key);
  const uint8_t* src = stage + key * kD + 16 * (tid & 3);
  uint8_t* dst0 = buf + key * 128 + (slot0 << 4);
  uint8_t* dst1 = buf + key * 128 + ((slot0 ^ 1) << 4);
#pragma unroll
  for (int m = 0; m < kD / 64; ++m) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + 64 * m);
    u32x4 lo, hi;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      lo[2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[d], 1.0f, false));
      lo[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[d], 1.0f, true));
      hi[2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[d + 2], 1.0f, false));
      hi[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[d + 2], 1.0f, true));
    }
    *reinterpret_cast<u32x4*>(dst0 + 8192 * m) = lo;
    *reinterpret_cast<u32x4*>(dst1 + 8192 * m) = hi;
  }
}

// Read an index-array entry that is the same for every lane of the wave
// through the scalar cache.  The index arrays are never written while the
// kernel runs; the compiler cannot prove that for reads after the first
// output stores and would otherwise use a vector load and a full wait.
__device__ __forceinline__ int32_t uniform_load(const int32_t* p, int i) {
  using const_i32 = const __attribute__((address_space(4))) int32_t;
  return *((const_i32*)p + __builtin_amdgcn_readfirstlane(i));
}

__device__ __forceinline__ int32_t page_count(int32_t L) {
  return L > 0 ? (L + kPage - 1) / kPage : 0;
}

// Multiply one accumulator tile (16 AGPRs) by alpha in place, through one
// temporary VGPR.  Written in assembly because the compiler would otherwise
// copy all 256 accumulator registers to VGPRs for this rarely taken step.
// The trailing s_nop covers an MFMA reading the tile right after.
__device__ __forceinline__ void scale_tile(f32x16& acc, float alpha) {
  float e[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) e[i] = acc[i];
  float tmp;
  asm volatile(
      "v_accvgpr_read_b32 %16, %0\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %0, %16\n\t"
      "v_accvgpr_read_b32 %16, %1\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %1, %16\n\t"
      "v_accvgpr_read_b32 %16, %2\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %2, %16\n\t"
      "v_accvgpr_read_b32 %16, %3\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %3, %16\n\t"
      "v_accvgpr_read_b32 %16, %4\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %4, %16\n\t"
      "v_accvgpr_read_b32 %16, %5\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %5, %16\n\t"
      "v_accvgpr_read_b32 %16, %6\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %6, %16\n\t"
      "v_accvgpr_read_b32 %16, %7\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %7, %16\n\t"
      "v_accvgpr_read_b32 %16, %8\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %8, %16\n\t"
      "v_accvgpr_read_b32 %16, %9\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %9, %16\n\t"
      "v_accvgpr_read_b32 %16, %10\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %10, %16\n\t"
      "v_accvgpr_read_b32 %16, %11\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %11, %16\n\t"
      "v_accvgpr_read_b32 %16, %12\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %12, %16\n\t"
      "v_accvgpr_read_b32 %16, %13\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %13, %16\n\t"
      "v_accvgpr_read_b32 %16, %14\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %14, %16\n\t"
      "v_accvgpr_read_b32 %16, %15\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %15, %16\n\t"
      "s_nop 1"
      : "+a"(e[0]), "+a"(e[1]), "+a"(e[2]), "+a"(e[3]),
        "+a"(e[4]), "+a"(e[5]), "+a"(e[6]), "+a"(e[7]),
        "+a"(e[8]), "+a"(e[9]), "+a"(e[10]), "+a"(e[11]),
        "+a"(e[12]), "+a"(e[13]), "+a"(e[14]), "+a"(e[15]),
        "=&v"(tmp)
      : "v"(alpha));
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = e[i];
}

// ---------------------------------------------------------------------------
// The two MFMA chains of a page are issued from inline assembly, one MFMA
// per statement, with compiler scheduling barriers between statements so
// that the order written here is the order issued:
//  * LDS operand reads for a later group of four MFMAs are issued before the
//    current group, so they are in flight behind its matrix work (left to
//    itself the compiler would sink every read next to its MFMA, since the
//    kernel sits at the 512-register limit);
//  * after every MFMA a payload slot runs caller code (VALU work of the
//    softmax) in the shadow of the matrix pipe, and after every group a hook
//    (the next page's global loads);
//  * the waits for the reads are statements that take the read registers
//    as in/out operands, so no use of them can be placed above the wait.
// Hazards the compiler cannot see are covered by hand: 2 wait states before
// each MFMA (a VALU write of an operand just before), and 24 after the last
// MFMA of a chain (MFMA result -> VALU or accumulator read; more than a
// 16-pass MFMA needs).
// ---------------------------------------------------------------------------
#define MLA_SB() __builtin_amdgcn_sched_barrier(0)

template <int N>
using ic = std::integral_constant<int, N>;

// pin(x): an empty volatile statement that claims to modify x, so that
// nothing computed from x can move above it (used for the lane id, so that
// per-lane offsets are recomputed where they are needed).
// keep(x): an empty volatile statement that reads x, so that x is computed
// before it.  Payload code hands its results to one: with the scheduling
// barriers around each slot that confines the payload to its slot
// (scheduling barriers alone do not stop sinking of pure arithmetic into
// later blocks).  Unlike pin(), it costs no copy and no wait state.
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void keep(float x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void keep(uint32_t x) { asm volatile("" ::"v"(x)); }

struct NoSlot {
  template <int N>
  __device__ __forceinline__ void operator()(ic<N>) const {}
};

// S^T MFMA with the accumulator in VGPRs (the output accumulator takes all
// 256 AGPRs); FIRST starts from zero.
template <bool FIRST>
__device__ __forceinline__ void mfma_s(f32x16& c, const bf16x8& a, const bf16x8& b) {
  if constexpr (FIRST)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                 : "=&v"(c)
                 : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                 : "+v"(c)
                 : "v"(a), "v"(b));
}

// O^T MFMA, accumulator tile in AGPRs.  FRESH: the weights p were just
// written by VALU instructions (packing), which need 2 wait states before an
// MFMA reads them.
template <bool FRESH = false>
__device__ __forceinline__ void mfma_o(f32x16& o, const bf16x8& v, const bf16x8& p) {
  if constexpr (FRESH)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
}

__device__ __forceinline__ void mfma_tail() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"); }

// Clears the output accumulators with one MFMA per tile (zero operands, zero
// accumulator input): 16 instructions instead of 256 register writes.  The
// first one waits out the VALU write of the zero operand.
__device__ __forceinline__ void zero_acc(f32x16 (&oacc)[kVTiles]) {
  const bf16x8 z = {};
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(oacc[0]) : "v"(z));
#pragma unroll
  for (int vt = 1; vt < kVTiles; ++vt)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(oacc[vt]) : "v"(z));
}

// S^T chain: one 16-byte K-operand read per MFMA, from a ring of kKRing
// operand slots.  The read for k-step ks+kKAhead is issued right after
// MFMA ks, into the slot MFMA ks-1 used (its operands were read when it
// issued, a full MFMA earlier); after every second MFMA one wait covers the
// reads of the next two -- so every read has at least kKAhead - 2 MFMAs to
// arrive.  (A single wave per SIMD issues at most one instruction per
// 4-cycle turn: the chain is kept to the instructions it needs.)
constexpr int kKRing = 9;
constexpr int kKAhead = kKRing - 1;

// K operand of k-step KS of the tile at byte offset TB: 16 bytes at
// a[KS % 4] + 8192 (KS / 4) + TB (column block KS / 4).  Column block 8 lies
// past the DS offset field (65535): its address is moved up by 32 KiB first.
template <int TB, int KS>
__device__ __forceinline__ void k_read(bf16x8& dst, const uint32_t (&a)[4]) {
  constexpr int OFF = 8192 * (KS / 4) + TB;
  if constexpr (OFF < 65536) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=&v"(dst) : "v"(a[KS % 4]), "i"(OFF));
  } else {
    uint32_t t;
    asm volatile("v_add_u32 %1, 0x8000, %2\n\tds_read_b128 %0, %1 offset:%3"
                 : "=&v"(dst), "=&v"(t)
                 : "v"(a[KS % 4]), "i"(OFF - 32768));
  }
}

// Wait until at most N LDS reads are outstanding (x is usable after it).  A
// plain wait instruction: the reads and their consumers are volatile
// statements, which keep their order around it, and an inline-assembly wait
// claiming to write x would cost a wait state before the MFMA reading x.
template <int N>
__device__ __forceinline__ void lgkm_wait() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
}

// Step KS of the S^T chain of the tile at TB: MFMA KS, payload slot KS, the
// read for KS + kKAhead, after an odd KS the wait for KS + 1 and KS + 2, and
// hook(KS / 4) after every fourth MFMA (the waits leave no read in flight
// across a hook only at the end of the chain, so hooks must not touch LDS
// reads).
template <int TB, int KS, typename Hook, typename Pay>
__device__ __forceinline__ void s_step(f32x16& sc, bf16x8 (&ring)[kKRing],
                                       const bf16x8 (&qreg)[kKSteps], const uint32_t (&a)[4],
                                       Hook& hook, Pay& pay) {
  mfma_s<KS == 0>(sc, ring[KS % kKRing], qreg[KS]);
  MLA_SB();
  pay(ic<KS>{});
  MLA_SB();
  if constexpr (KS + kKAhead < kKSteps) k_read<TB, KS + kKAhead>(ring[(KS + kKAhead) % kKRing], a);
  MLA_SB();
  if constexpr (KS + 1 == kKSteps) {
    mfma_tail();
  } else if constexpr (KS % 2 == 1) {
    // reads issued after the ones for KS + 1 and KS + 2
    constexpr int last = (KS + kKAhead < kKSteps) ? KS + kKAhead : kKSteps - 1;
    constexpr int need = (KS + 2 < kKSteps) ? KS + 2 : KS + 1;
    lgkm_wait<last - need>();
  }
  MLA_SB();
  if constexpr (KS % 4 == 3) {
    hook(ic<KS / 4>{});
    MLA_SB();
  }
}

template <int TB, typename Hook, typename Pay, int... KS>
__device__ __forceinline__ void s_steps(f32x16& sc, bf16x8 (&ring)[kKRing],
                                        const bf16x8 (&qreg)[kKSteps], const uint32_t (&a)[4],
                                        Hook& hook, Pay& pay, std::integer_sequence<int, KS...>) {
  (s_step<TB, KS>(sc, ring, qreg, a, hook, pay), ...);
}

template <int TB, int... KS>
__device__ __forceinline__ void s_prologue(bf16x8 (&ring)[kKRing], const uint32_t (&a)[4],
                                           std::integer_sequence<int, KS...>) {
  (k_read<TB, KS>(ring[KS], a), ...);
}

// S^T for the 32-key tile at byte offset TB of the page: 36 MFMAs.
// pay(ic<s>) runs after MFMA s (0..35), hook(ic<G>) after MFMA 4G+3.
// ka0 = page + the lane's K offset for 16-byte chunk 0 (LDS byte address);
// chunk i of the lane's k-step is at ka0 ^ 32 i (see the swizzle above).
template <int TB, typename Hook, typename Pay>
__device__ __forceinline__ void score_tile(f32x16& sc, uint32_t ka0,
                                           const bf16x8 (&qreg)[kKSteps], Hook&& hook,
                                           Pay&& pay) {
  const uint32_t a[4] = {ka0, ka0 ^ 32u, ka0 ^ 64u, ka0 ^ 96u};
  bf16x8 ring[kKRing];
  s_prologue<TB>(ring, a, std::make_integer_sequence<int, kKAhead>{});
  lgkm_wait<kKAhead - 2>();  // k-steps 0 and 1
  MLA_SB();
  s_steps<TB>(sc, ring, qreg, a, hook, pay, std::make_integer_sequence<int, kKSteps>{});
}

// The output chain of a 32-key tile: 32 MFMAs (16 accumulator tiles x two
// 16-key steps) in 8 groups of 4.  V^T operands come from kPvRing rotating
// sets: group b uses set b % kPvRing and issues the reads of group
// b + kPvRing - 1 into the set group b - 1 used, then waits until group
// b + 1's set has landed; each read has kPvRing - 1 groups (about 270 cycles)
// of matrix work to arrive.  An operand is two transposing 8-byte
// reads (keys kb..kb+3 and kb+4..kb+7 of the lane half) at va[0][par] + off
// and va[1][par] + off.
constexpr int kPvBlocks = 2 * kVTiles / 4;  // 8 groups of 4 MFMAs per 32-key tile
constexpr int kPvRing = 3;                  // operand sets; reads run kPvRing - 1 groups ahead

// LDS offsets (relative to va) of group nb's reads: MFMA i = 4 nb + j has
// u = i / 16 (keys 8u..8u+7 of the lane half) and vt = i % 16; MFMAs j = 0, 1
// share column block vt/2 (off0), j = 2, 3 the next one (off1).
template <int T, int NB>
struct PvOff {
  static constexpr int n0 = 4 * NB, nu = n0 / kVTiles, nvt = n0 % kVTiles;
  static constexpr int row = (32 * T + 8 * nu) * 128;
  static constexpr int off0 = row + 8192 * (nvt >> 1);
  static constexpr int off1 = row + 8192 * ((nvt + 2) >> 1);
};

struct VSet {
  bf16x4 lo[4], hi[4];
};

template <int T, int NB>
__device__ __forceinline__ void v_reads(VSet& s, const uint32_t (&va)[2][2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %[l0], %[a00] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[h0], %[a10] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[l1], %[a01] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[h1], %[a11] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[l2], %[a00] offset:%[o1]\n\t"
      "ds_read_b64_tr_b16 %[h2], %[a10] offset:%[o1]\n\t"
      "ds_read_b64_tr_b16 %[l3], %[a01] offset:%[o1]\n\t"
      "ds_read_b64_tr_b16 %[h3], %[a11] offset:%[o1]"
      : [l0] "=&v"(s.lo[0]), [l1] "=&v"(s.lo[1]), [l2] "=&v"(s.lo[2]), [l3] "=&v"(s.lo[3]),
        [h0] "=&v"(s.hi[0]), [h1] "=&v"(s.hi[1]), [h2] "=&v"(s.hi[2]), [h3] "=&v"(s.hi[3])
      : [a00] "v"(va[0][0]), [a10] "v"(va[1][0]), [a01] "v"(va[0][1]), [a11] "v"(va[1][1]),
        [o0] "i"(PvOff<T, NB>::off0), [o1] "i"(PvOff<T, NB>::off1));
}

// Half H of v_reads (operands 2H and 2H + 1 of the set).
template <int T, int NB, int H>
__device__ __forceinline__ void v_reads_half(VSet& s, const uint32_t (&va)[2][2]) {
  constexpr int o = H == 0 ? PvOff<T, NB>::off0 : PvOff<T, NB>::off1;
  asm volatile(
      "ds_read_b64_tr_b16 %[l0], %[a00] offset:%[o]\n\t"
      "ds_read_b64_tr_b16 %[h0], %[a10] offset:%[o]\n\t"
      "ds_read_b64_tr_b16 %[l1], %[a01] offset:%[o]\n\t"
      "ds_read_b64_tr_b16 %[h1], %[a11] offset:%[o]"
      : [l0] "=&v"(s.lo[2 * H]), [l1] "=&v"(s.lo[2 * H + 1]), [h0] "=&v"(s.hi[2 * H]),
        [h1] "=&v"(s.hi[2 * H + 1])
      : [a00] "v"(va[0][0]), [a10] "v"(va[1][0]), [a01] "v"(va[0][1]), [a11] "v"(va[1][1]),
        [o] "i"(o));
}

// Wait until at most N LDS reads are outstanding; s becomes usable after it.
template <int N>
__device__ __forceinline__ void v_wait(VSet&) {
  lgkm_wait<N>();
}

// MFMA J of group B of an output chain, then payload slot 4B+J.
template <int B, int J, typename Pay>
__device__ __forceinline__ void pv_mfma(f32x16 (&oacc)[kVTiles], const VSet& s,
                                        const bf16x8 (&pop)[2], Pay& pay) {
  constexpr int u = (4 * B) / kVTiles, vt = (4 * B) % kVTiles + J;
  mfma_o<(4 * B + J) % kVTiles == 0>(
      oacc[vt], __builtin_shufflevector(s.lo[J], s.hi[J], 0, 1, 2, 3, 4, 5, 6, 7), pop[u]);
  MLA_SB();
  pay(ic<4 * B + J>{});
  MLA_SB();
}

// The reads for group B + kAhead go out in two halves, before MFMAs 0 and 3
// of the group, so that no gap between two MFMAs holds more than a few
// instructions (the payload of slot 4B + 1 sits between MFMAs 1 and 2).
template <int T, int B, typename Hook, typename Pay, int... J>
__device__ __forceinline__ void pv_group(f32x16 (&oacc)[kVTiles], VSet (&ring)[kPvRing],
                                         const bf16x8 (&pop)[2], const uint32_t (&va)[2][2],
                                         Hook& hook, Pay& pay, std::integer_sequence<int, J...>) {
  constexpr int kAhead = kPvRing - 1;
  constexpr bool kRead = B + kAhead < kPvBlocks;
  if constexpr (kRead) v_reads_half<T, B + kAhead, 0>(ring[(B + kAhead) % kPvRing], va);
  MLA_SB();
  pv_mfma<B, 0>(oacc, ring[B % kPvRing], pop, pay);
  pv_mfma<B, 1>(oacc, ring[B % kPvRing], pop, pay);
  pv_mfma<B, 2>(oacc, ring[B % kPvRing], pop, pay);
  if constexpr (kRead) v_reads_half<T, B + kAhead, 1>(ring[(B + kAhead) % kPvRing], va);
  MLA_SB();
  pv_mfma<B, 3>(oacc, ring[B % kPvRing], pop, pay);
  if constexpr (B + 1 < kPvBlocks) {
    // reads issued after group B+1's: groups B+2 .. min(B+kAhead, last)
    constexpr int last = (B + kAhead < kPvBlocks) ? B + kAhead : kPvBlocks - 1;
    v_wait<8 * (last - (B + 1))>(ring[(B + 1) % kPvRing]);
  } else {
    mfma_tail();
  }
  MLA_SB();
  hook(ic<B>{});
  MLA_SB();
}

template <int T, typename Hook, typename Pay, int... B>
__device__ __forceinline__ void pv_chain(f32x16 (&oacc)[kVTiles], VSet (&ring)[kPvRing],
                                         const bf16x8 (&pop)[2], const uint32_t (&va)[2][2],
                                         Hook& hook, Pay& pay, std::integer_sequence<int, B...>) {
  (pv_group<T, B>(oacc, ring, pop, va, hook, pay, std::make_integer_sequence<int, 4>{}), ...);
}

template <int T, int... B>
__device__ __forceinline__ void pv_prologue(VSet (&ring)[kPvRing], const uint32_t (&va)[2][2],
                                            std::integer_sequence<int, B...>) {
  (v_reads<T, B>(ring[B], va), ...);
}

// O^T += V^T P^T for 32-key tile T: 32 MFMAs.  pay(ic<s>) runs after MFMA s
// (0..31), hook(ic<B>) after group B.  va0 = page + the lane's V offset for
// (e, par) = (0, 0); the others follow from the swizzle:
// (0, 1) = va0 ^ 64, (1, 0) = (va0 + 512) ^ 32, (1, 1) = that ^ 64.
template <int T, typename Hook, typename Pay>
__device__ __forceinline__ void pv_tile(f32x16 (&oacc)[kVTiles], const bf16x8 (&pop)[2],
                                        uint32_t va0, Hook&& hook, Pay&& pay) {
  const uint32_t va10 = (va0 + 512u) ^ 32u;
  const uint32_t va[2][2] = {{va0, va0 ^ 64u}, {va10, va10 ^ 64u}};
  VSet ring[kPvRing];
  pv_prologue<T>(ring, va, std::make_integer_sequence<int, kPvRing - 1>{});
  v_wait<8 * (kPvRing - 2)>(ring[0]);
  MLA_SB();
  pv_chain<T>(oacc, ring, pop, va, hook, pay, std::make_integer_sequence<int, kPvBlocks>{});
}

// ---- the second score tile and the first output tile as one chain ----------
// On its own an output tile is bound by its transposing V^T reads (two per
// MFMA) and a score tile by the matrix pipe (one K read per MFMA).  Mixing
// the two, slot by slot, keeps the matrix pipe busy through both.  Slot s
// holds one MFMA: the first kCPrefix slots are score MFMAs of tile 1 (while
// the weights of tile 0 are computed in their shadow), the next kCMixed
// slots spread the remaining score MFMAs evenly among output MFMAs of tile
// 0, and the rest are output MFMAs (in whose shadow the row max and the
// first weights of tile 1 are computed).  Every slot reads 16 bytes of
// operand per lane (one K read, or two 8-byte V^T reads), kCAhead slots
// before its MFMA; the reads are waited for two slots at a time.
constexpr int kCSlots = kKSteps + 2 * kVTiles;  // 36 score + 32 output MFMAs
constexpr int kCPrefix = 9;
constexpr int kCMixed = 50;
constexpr int kCAhead = 8;

__host__ __device__ constexpr bool cs_is_s(int s) {
  if (s < kCPrefix) return true;
  if (s >= kCPrefix + kCMixed) return false;
  const int t = s - kCPrefix, n = kKSteps - kCPrefix;
  return (t + 1) * n / kCMixed != t * n / kCMixed;
}
// index of slot s's MFMA within its own chain (k-step, or output MFMA)
__host__ __device__ constexpr int cs_index(int s) {
  int c = 0;
  for (int u = 0; u < s; ++u) c += (cs_is_s(u) == cs_is_s(s)) ? 1 : 0;
  return c;
}
__host__ __device__ constexpr int cs_reads(int s) { return cs_is_s(s) ? 1 : 2; }
// The wait before slot s (s even) covers slots s and s + 1: LDS reads issued
// after slot s + 1's, i.e. those of slots s+2 .. s+kCAhead-1 (the reads of
// slots up to s - 1 + kCAhead are out by then).
__host__ __device__ constexpr int cs_wait(int s) {
  int n = 0;
  for (int u = s + 2; u < s + kCAhead && u < kCSlots; ++u) n += cs_reads(u);
  return n;
}
__host__ __device__ constexpr int cs_slot_of(bool score, int index) {
  for (int s = 0; s < kCSlots; ++s)
    if (cs_is_s(s) == score && cs_index(s) == index) return s;
  return -1;
}
__host__ __device__ constexpr bool cs_layout_ok() {
  int ns = 0, wmax = 0;
  for (int s = 0; s < kCSlots; ++s) {
    ns += cs_is_s(s) ? 1 : 0;
    if (s % 2 == 0) wmax = cs_wait(s) > wmax ? cs_wait(s) : wmax;
  }
  return ns == kKSteps && wmax <= 15;
}
static_assert(cs_layout_ok() && kCSlots % 2 == 0,
              "combined chain: 36 score slots, waits within lgkmcnt range");
constexpr int kCLastScore = cs_slot_of(true, kKSteps - 1);  // 58
constexpr int kCFirstOut = cs_slot_of(false, 0);            // 9
// 43: the first output MFMA on keys 8..15 of each lane half (weights pop[1])
constexpr int kCOutU1 = cs_slot_of(false, kVTiles);
static_assert(kCLastScore == 58 && kCFirstOut == 9 && kCOutU1 == 43,
              "the page loop's payload slots are placed for this layout");

struct COps {
  bf16x8 k[kCSlots];            // score slots
  bf16x4 lo[kCSlots], hi[kCSlots];  // output slots
};

// Operand reads of slot S: the K read of tile 1 (byte offset 32 * 128), or
// the two V^T reads of output MFMA j of tile 0 (accumulator tile j % 16,
// keys 8 (j / 16) .. +7 of the lane half; see pv_tile for the addresses).
template <int S>
__device__ __forceinline__ void c_read(COps& op, const uint32_t (&a)[4],
                                       const uint32_t (&va)[2][2]) {
  if constexpr (cs_is_s(S)) {
    k_read<32 * 128, cs_index(S)>(op.k[S], a);
  } else {
    constexpr int j = cs_index(S), vt = j % kVTiles, u = j / kVTiles;
    constexpr int off = 8 * u * 128 + 8192 * (vt >> 1);
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2 offset:%4\n\t"
        "ds_read_b64_tr_b16 %1, %3 offset:%4"
        : "=&v"(op.lo[S]), "=&v"(op.hi[S])
        : "v"(va[0][vt & 1]), "v"(va[1][vt & 1]), "i"(off));
  }
}

template <int S>
__device__ __forceinline__ void c_wait() {
  lgkm_wait<cs_wait(S)>();
}

// Slot S: its MFMA, pay(ic<S>) in its shadow, the reads of slot S + kCAhead,
// after an odd slot the wait for the next two, then hook(ic<S>).
template <int S, typename Hook, typename Pay>
__device__ __forceinline__ void c_step(f32x16& sc, f32x16 (&oacc)[kVTiles], COps& op,
                                       const bf16x8 (&pop)[2], const bf16x8 (&qreg)[kKSteps],
                                       const uint32_t (&a)[4], const uint32_t (&va)[2][2],
                                       Hook& hook, Pay& pay) {
  if constexpr (cs_is_s(S)) {
    constexpr int ks = cs_index(S);
    mfma_s<ks == 0>(sc, op.k[S], qreg[ks]);
  } else {
    constexpr int j = cs_index(S);
    mfma_o<j % kVTiles == 0>(oacc[j % kVTiles],
                             __builtin_shufflevector(op.lo[S], op.hi[S], 0, 1, 2, 3, 4, 5, 6, 7),
                             pop[j / kVTiles]);
  }
  MLA_SB();
  pay(ic<S>{});
  MLA_SB();
  if constexpr (S + kCAhead < kCSlots) c_read<S + kCAhead>(op, a, va);
  MLA_SB();
  if constexpr (S + 1 == kCSlots)
    mfma_tail();
  else if constexpr (S % 2 == 1)
    c_wait<S + 1>();
  MLA_SB();
  hook(ic<S>{});
  MLA_SB();
}

template <typename Hook, typename Pay, int... S>
__device__ __forceinline__ void c_steps(f32x16& sc, f32x16 (&oacc)[kVTiles], COps& op,
                                        const bf16x8 (&pop)[2], const bf16x8 (&qreg)[kKSteps],
                                        const uint32_t (&a)[4], const uint32_t (&va)[2][2],
                                        Hook& hook, Pay& pay, std::integer_sequence<int, S...>) {
  (c_step<S>(sc, oacc, op, pop, qreg, a, va, hook, pay), ...);
}

template <int... S>
__device__ __forceinline__ void c_prologue(COps& op, const uint32_t (&a)[4],
                                           const uint32_t (&va)[2][2],
                                           std::integer_sequence<int, S...>) {
  (c_read<S>(op, a, va), ...);
}

// S^T of tile 1 into sc and O^T += V^T P^T for tile 0 (pop: its weights,
// pop[0] used from slot kCFirstOut, pop[1] from slot kCOutU1), ka0 / va0 as
// for score_tile / pv_tile.
template <typename Hook, typename Pay>
__device__ __forceinline__ void combined_chain(f32x16& sc, f32x16 (&oacc)[kVTiles],
                                               const bf16x8 (&pop)[2],
                                               const bf16x8 (&qreg)[kKSteps], uint32_t ka0,
                                               uint32_t va0, Hook&& hook, Pay&& pay) {
  const uint32_t a[4] = {ka0, ka0 ^ 32u, ka0 ^ 64u, ka0 ^ 96u};
  const uint32_t va10 = (va0 + 512u) ^ 32u;
  const uint32_t va[2][2] = {{va0, va0 ^ 64u}, {va10, va10 ^ 64u}};
  COps op;
  c_prologue(op, a, va, std::make_integer_sequence<int, kCAhead>{});
  c_wait<0>();
  MLA_SB();
  c_steps(sc, oacc, op, pop, qreg, a, va, hook, pay, std::make_integer_sequence<int, kCSlots>{});
}

// Max / sum over the two lane halves (which hold the same query row's other
// keys), exchanged with v_permlane32_swap.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-lane constants of the page loop.  The loop runs at the 512-register
// limit, so these are recomputed from a pinned lane id (a few VALU
// instructions) where they are needed rather than held in registers, which
// the compiler would spill and reload with a wait on all vector memory.
struct LaneOffsets {
  uint32_t k;     // S^T A operand: LDS offset of the lane's 16-byte chunk 0
  uint32_t v;     // V^T A operand: LDS offset for (e, par) = (0, 0)
  uint32_t load;  // bf16 page load, key group = wave: global (= LDS source) offset
};

__device__ __forceinline__ uint32_t pinned_lane() {
  uint32_t l = lane_id();
  pin(l);
  return l;
}

__device__ __forceinline__ LaneOffsets lane_offsets(uint32_t lane, int wave) {
  LaneOffsets o;
  const int n = lane & 31, h = lane >> 5;
  // S^T A operand: lane (m = n, h) reads key 32t + sigma(m) with
  // sigma(8q + 4g + t') = 16g + 4q + t', global chunk 2ks + h, i.e. column
  // block ks/4, chunk 2(ks%4) + h of the block.  Keys 32 apart share the
  // swizzle, so tile 1 is tile 0 plus 32 rows of 128 bytes; chunk i of the
  // lane's k-step is at o.k ^ 32 i.
  const int sig = 16 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
  o.k = sig * 128 + ((h ^ chunk_swz(sig)) << 4);
  // V^T A operand via ds_read_b64_tr_b16: in the 16-lane block (c16, s16)
  // of half h, source lane s16 addresses key kb + 4e + s16/4 (kb a multiple
  // of 8 with bit 4 = h), columns 32vt + 16c16 + 4(s16%4) .. +3; the block
  // then holds column 32vt + 16c16 + s16 of keys kb+4e .. kb+4e+3.
  const int s16 = lane & 15, c16 = (lane >> 4) & 1, a = s16 >> 2;
  const int cc = 2 * c16 + ((s16 >> 1) & 1);
  o.v = (16 * h + a) * 128 + ((cc ^ (4 * (a >> 1) + h)) << 4) + 8 * (s16 & 1);
  // Page loads: key i/8 of the group, chunk slot i%8 <- source chunk
  // (i%8) ^ (4 bit4(i) + 2 bit5(i) + bit1(wave)).
  o.load = wave * (8 * kRowBytes) + (lane >> 3) * kRowBytes +
           16 * ((lane & 7) ^ (4 * ((lane >> 4) & 1) + 2 * ((lane >> 5) & 1) + ((wave >> 1) & 1)));
  return o;
}

// Bytes of LDS each wave has for staging its output rows (outside the page
// buffers, so no other wave is ever waiting on them).
constexpr int kStageBytes = 4096;

// Values 4G .. 4G+3 of an accumulator tile to LDS, straight from the
// accumulator registers.
template <int G>
__device__ __forceinline__ void stage_quad(const f32x16& tile, uint32_t addr) {
  const f32x4 quad = __builtin_shufflevector(tile, tile, 4 * G, 4 * G + 1, 4 * G + 2, 4 * G + 3);
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "a"(quad) : "memory");
}

// Write this wave's 32 rows of o * scale, as rows of 512 values, to dst (row
// r at dst + r * 512), in fp32 (T = float: the partial state of a piece) or
// bf16 (T = uint16_t: the output of an unsplit request).  The accumulators
// hold O^T (lane (n, h): row n, 16 values per tile), so direct stores would
// write 16-byte pieces of 32 rows per instruction.  Instead each tile (32
// columns, 128 bytes of each row in fp32) goes to the wave's own LDS area
// straight from the accumulator registers, unscaled (the 16-byte chunk c of
// row n at c ^ (n % 8), which spreads writes and reads over the banks), and
// leaves row-major: lane i reads 4 values of row 8 qq + i / 8, scales them by
// that row's scale (taken from the lane that computed it) and stores them,
// so that a store instruction covers 8 rows x 128 bytes (fp32) or 64 bytes
// (bf16).  Few registers are live at a time, which leaves the next piece's
// queries room to stay in registers across the epilogue.  FULL: all 32 rows
// exist (no row checks).
template <typename T, bool FULL>
__device__ __forceinline__ void store_rows(const f32x16 (&oacc)[kVTiles], float scale,
                                           uint8_t* stage, T* dst, int row0, int rows,
                                           uint32_t lane) {
  constexpr bool kBf16 = sizeof(T) == 2;
  const int n = lane & 31, h = lane >> 5, j = lane & 7;
  const uint32_t sbase = (uint32_t)(uintptr_t)LDS_PTR(uint8_t, stage);
  uint32_t wa[4];  // LDS addresses of this lane's 4 chunks of a tile (chunk 2g + h of row n)
#pragma unroll
  for (int g = 0; g < 4; ++g) wa[g] = sbase + n * 128 + (((2 * g + h) ^ (n & 7)) << 4);
  float rs[4];
  T* rowp[4];
  const uint4* ra[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int row = 8 * qq + (int)(lane >> 3);
    rs[qq] = __shfl(scale, row);
    ra[qq] = reinterpret_cast<const uint4*>(stage + row * 128 + ((j ^ (row & 7)) << 4));
    rowp[qq] = dst + (int64_t)(row0 + row) * kDv + 4 * j;
  }
  // Tile p + 1 goes to LDS and is read back while tile p is scaled and
  // stored: a wave's LDS operations run in order, so the writes of tile p + 1
  // land after the reads of tile p have taken the old contents.
  auto stage_tile = [&](const f32x16& tile) {
    stage_quad<0>(tile, wa[0]);
    stage_quad<1>(tile, wa[1]);
    stage_quad<2>(tile, wa[2]);
    stage_quad<3>(tile, wa[3]);
  };
  uint4 cur[4], nxt[4];
  stage_tile(oacc[0]);
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) cur[qq] = *ra[qq];
#pragma unroll
  for (int p = 0; p < kVTiles; ++p) {
    if (p + 1 < kVTiles) {
      stage_tile(oacc[p + 1]);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) nxt[qq] = *ra[qq];
    }
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const float4 v = __builtin_bit_cast(float4, cur[qq]);
      const float x0 = v.x * rs[qq], x1 = v.y * rs[qq], x2 = v.z * rs[qq], x3 = v.w * rs[qq];
      if (FULL || row0 + 8 * qq + (int)(lane >> 3) < rows) {
        if constexpr (kBf16) {
          const uint32_t lo =
              __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x0, x1}, bf16x2));
          const uint32_t hi =
              __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x2, x3}, bf16x2));
          *reinterpret_cast<uint2*>(rowp[qq] + 32 * p) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<float4*>(rowp[qq] + 32 * p) = make_float4(x0, x1, x2, x3);
        }
      }
    }
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) cur[qq] = nxt[qq];
    __builtin_amdgcn_sched_barrier(0);  // two tiles of registers live at a time
  }
}

// The e4m3-query decode kernel's launch (decode_q8.hip).
void launch_decode_q8(dim3 grid, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop,
                      const uint8_t* q, const uint8_t* kv, const int32_t* block_table,
                      const int32_t* seq_lens, const int32_t* tile_plan,
                      const int32_t* split_indptr, const float* kv_descale,
                      const float* q_descale, uint16_t* partial_o, float* partial_lse,
                      uint16_t* out, float* lse, const DecodeParams& p);

}  // namespace mla
