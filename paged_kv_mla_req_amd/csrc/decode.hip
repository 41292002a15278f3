// MLA decode over a paged latent cache, split along the KV sequence.
//
// What it computes: for each request b and query row r (token i, head h),
// softmax attention of the 576-wide absorbed query over the request's latent
// rows 0..L_b-1 (bottom-right causal for q_len > 1), with V the first 512
// columns of the same latent row.  This is what the FlashMLA backend page's
// forward_decode (and the target-verify branch of forward_extend) asks of
// flash_mla_with_kvcache: k_cache viewed as [-1, 64, 1, 576],
// head_dim_v = kv_lora_rank, softmax_scale = layer.scaling, causal = True,
// cache_seqlens = prefix + draft tokens for verify.
//
// How (gfx950):
//  * One work-group of 4 waves per planner part (grid.x) and per block of 128
//    query rows (grid.y).  A part is a contiguous run of (request, page)
//    pairs; the work-group streams those pages once, and every page is shared
//    by all rows of the request (all heads share one latent row per token).
//  * Pages move HBM -> LDS with direct-to-LDS 16-byte buffer loads
//    (buffer_load_dwordx4 ... lds): 72 loads of 1 KiB per 72 KiB page,
//    double buffered, so the next page streams in while the current one is
//    used.  In LDS a page is 9 column blocks of 8 KiB (64 columns of all 64
//    keys, 128 bytes per key); the 16-byte chunk c of key k inside a block
//    sits at chunk c ^ swz(k), swz(k) = 4*bit1(k) + 2*bit2(k) + bit4(k).
//    With that swizzle both LDS read patterns below (16-byte key reads and
//    transposing value reads) touch every bank once per half-wave, and every
//    1 KiB load has one of two per-lane source offsets.
//  * Each wave owns 32 query rows and keeps them in registers (MFMA B
//    operand, 144 VGPRs).  Scores are computed transposed, S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16: the key rows of the A operand are permuted so
//    that lane (row n, half h) ends up holding 16 consecutive keys of each
//    32-key tile for its own query row.  Row max and row sum are then
//    in-lane plus one exchange between the two lane halves.
//  * The output is also kept transposed, O^T += V^T P^T: P (in registers, B
//    operand) needs no data movement, and V^T comes straight from the
//    key-major page with ds_read_b64_tr_b16 (each lane receives one value
//    column of four consecutive keys).  O^T is 16 accumulator tiles.
//  * Online softmax in base 2 with a lazy rescale: the running max moves
//    only when a new score exceeds it by more than 8 (so p <= 2^8), which
//    keeps the 256-register rescale off the common path.
//  * Epilogue: an unsplit request writes bf16 o and fp32 lse; a piece of a
//    split request writes its fp32 (o, lse) to the partial slot the planner
//    assigned, for mla_merge_states.
//  * fp8 cache (FlashMLA backend page, forward_decode fp8 branch; AITER
//    helper page, forward_decode_vectorized_5d): the page holds e4m3fn bytes
//    whose latent value is byte * delta, delta one per-tensor scale read from
//    device memory.  A page (36 KiB) lands in one of two LDS staging buffers
//    and the work-group converts it to bf16 -- exact, since every e4m3 value
//    is a bf16 value -- into the single 72 KiB compute buffer, in the layout
//    above; the MFMA work is then the bf16 work.  delta scales the scores
//    (folded into the softmax scale, with its sign moved onto q) and the
//    output.
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
constexpr int kCLastScore = cs_slot_of(true, kKSteps - 1);  // 54
constexpr int kCFirstOut = cs_slot_of(false, 0);            // 13
constexpr int kCOutU1 = cs_slot_of(false, kVTiles);         // 48: first MFMA on keys 16..31

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

// ---- fp8 query (e4m3 codes) over an e4m3 cache ------------------------------
// The scores run on v_mfma_f32_32x32x64_f8f6f4 (both operands e4m3, 64
// columns per MFMA: 9 per 32-key tile instead of 36), straight from the
// page's e4m3 bytes in LDS; the output contraction stays bf16 (the weights p
// keep bf16 precision; V comes from the exact e4m3 -> bf16 conversion).
//
// LDS for this variant: the bf16 V page (8 column blocks of 8 KiB, the
// layout of the bf16 page above) at offset 0, and two e4m3 staging buffers
// from kQ8Stage on.  A staging buffer is 9 column blocks of 4 KiB (64
// columns of all 64 keys, 64 bytes per key); the 16-byte chunk c of key k in
// a block sits at slot c ^ f8_swz(k), f8_swz(k) = bit2(k) + 2 bit4(k), so
// that the score operand reads (32 keys, two chunks each) touch every bank
// once per 16 lanes.
//
// V needs no pass of its own: every wave reads the whole page as score
// operands anyway, so while its score MFMAs run wave w converts the operand
// registers of column blocks 2w and 2w + 1 (both key tiles) to bf16 and
// writes them to the V page; one barrier (LDS only) between the score and
// the output phase publishes them.
constexpr int kKSteps8 = kD / 64;            // 9 fp8 k-steps of 64 columns
constexpr int kQ8Stage = kDv * kPage * 2;    // 65536: staging buffers after the V page
constexpr int kK8Ahead = 3;                  // operand reads run 3 MFMAs ahead
constexpr int kK8Ring = kK8Ahead + 1;
static_assert(kQ8Stage + 2 * kPageBytesF8 <= 2 * kPageBytes, "q8 LDS layout fits the page buffers");

typedef uint32_t u32x8 __attribute__((__vector_size__(8 * sizeof(uint32_t))));

__device__ __forceinline__ int f8_swz(int k) { return ((k >> 2) & 1) + 2 * ((k >> 4) & 1); }

// Load K of wave w (K < 9) of an e4m3 page into the staging layout above:
// column block K, keys 16w .. 16w + 15; lane i writes slot i % 4 of key
// 16w + i / 4 from global chunk (i % 4) ^ f8_swz(key) (voff, per lane; the
// column block is the immediate offset, which moves the LDS destination
// too).
template <int K>
__device__ __forceinline__ void issue_one_load_q8(__amdgpu_buffer_rsrc_t rsrc, uint8_t* stage,
                                                  int wave, uint32_t voff) {
  constexpr int imm = 64 * K;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, LDS_PTR(void, stage + 4096 * K + 1024 * wave - imm), 16, voff, 0, imm, kStreamLoad);
}

template <int... K>
__device__ __forceinline__ void issue_loads_q8(std::integer_sequence<int, K...>,
                                               __amdgpu_buffer_rsrc_t rsrc, uint8_t* stage,
                                               int wave, uint32_t voff) {
  (issue_one_load_q8<K>(rsrc, stage, wave, voff), ...);
}

__device__ __forceinline__ uint32_t q8_load_offset(uint32_t lane, int wave) {
  const int key = 16 * wave + (int)(lane >> 2);
  return key * kD + 16 * (((int)lane & 3) ^ f8_swz(key));
}

// Per-lane LDS offsets of the q8 page loop (lane (m, h), m = lane % 32):
//  k: score A operand, key sigma(m) (as in lane_offsets), chunk 2h of the
//     column block; chunk 2h + 1 is at k ^ 16;
//  d: V conversion, bf16 chunk 4h of key sigma(m) in its column block;
//     chunks 4h + i are at d ^ 16 i.
struct Q8Offsets {
  uint32_t k, d;
};
__device__ __forceinline__ Q8Offsets q8_offsets(uint32_t lane) {
  const int n = lane & 31, h = lane >> 5;
  const int sig = 16 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
  Q8Offsets o;
  o.k = sig * 64 + (((2 * h) ^ f8_swz(sig)) << 4);
  o.d = sig * 128 + (((4 * h) ^ chunk_swz(sig)) << 4);
  return o;
}

template <bool FIRST>
__device__ __forceinline__ void mfma_s8(f32x16& c, const u32x8& a, const u32x8& b) {
  if constexpr (FIRST)
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}

struct K8 {
  u32x4 lo, hi;  // columns 32h .. 32h + 15 and 32h + 16 .. 32h + 31 of the block
};

// Score operand of step S (tile S / 9, column block S % 9): two 16-byte reads.
template <int S>
__device__ __forceinline__ void k8_read(K8& dst, uint32_t a0, uint32_t a1) {
  constexpr int OFF = 4096 * (S % kKSteps8) + 2048 * (S / kKSteps8);
  asm volatile("ds_read_b128 %0, %2 offset:%4\n\tds_read_b128 %1, %3 offset:%4"
               : "=&v"(dst.lo), "=&v"(dst.hi)
               : "v"(a0), "v"(a1), "i"(OFF));
}

template <bool HI>
__device__ __forceinline__ uint32_t cvt_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// the four e4m3 values of w to bf16
__device__ __forceinline__ uint2 cvt_bf16x4(uint32_t w) {
  return make_uint2(cvt_bf16x2<false>(w), cvt_bf16x2<true>(w));
}
// 8 e4m3 values (words w0, w1) to one 16-byte chunk of bf16
__device__ __forceinline__ u32x4 cvt_chunk(uint32_t w0, uint32_t w1) {
  const uint2 a = cvt_bf16x4(w0), b = cvt_bf16x4(w1);
  return (u32x4){a.x, a.y, b.x, b.y};
}

// The 32 e4m3 values of operand r (step S: key tile S / 9, column block
// S % 9) to bf16, written to the V page as the lane's 4 chunks.  Exact.
template <int S>
__device__ __forceinline__ void k8_convert(const K8& r, const uint32_t (&d)[4]) {
  constexpr int OFF = 8192 * (S % kKSteps8) + 4096 * (S / kKSteps8);
  const u32x4 c0 = cvt_chunk(r.lo[0], r.lo[1]), c1 = cvt_chunk(r.lo[2], r.lo[3]);
  const u32x4 c2 = cvt_chunk(r.hi[0], r.hi[1]), c3 = cvt_chunk(r.hi[2], r.hi[3]);
  asm volatile(
      "ds_write_b128 %0, %4 offset:%8\n\t"
      "ds_write_b128 %1, %5 offset:%8\n\t"
      "ds_write_b128 %2, %6 offset:%8\n\t"
      "ds_write_b128 %3, %7 offset:%8" ::"v"(d[0]),
      "v"(d[1]), "v"(d[2]), "v"(d[3]), "v"(c0), "v"(c1), "v"(c2), "v"(c3), "i"(OFF));
}

// Step S of the 18-step score chain (tiles 0 and 1 back to back): MFMA S,
// pay(ic<S>), wave `conv`'s conversion of its column blocks, the operand read
// for S + kK8Ahead, the wait for S + 1 (the conversion writes, which also
// count, only make it wait a little longer), hook(ic<S>).
template <int S, typename Hook, typename Pay>
__device__ __forceinline__ void s8_step(f32x16& sc0, f32x16& sc1, K8 (&ring)[kK8Ring],
                                        const u32x8 (&qreg)[kKSteps8], uint32_t a0, uint32_t a1,
                                        const uint32_t (&d)[4], int conv, Hook& hook, Pay& pay) {
  constexpr int ks = S % kKSteps8, N = 2 * kKSteps8;
  const K8& r = ring[S % kK8Ring];
  const u32x8 a = __builtin_shufflevector(r.lo, r.hi, 0, 1, 2, 3, 4, 5, 6, 7);
  if constexpr (S < kKSteps8)
    mfma_s8<ks == 0>(sc0, a, qreg[ks]);
  else
    mfma_s8<ks == 0>(sc1, a, qreg[ks]);
  MLA_SB();
  pay(ic<S>{});
  MLA_SB();
  if constexpr (ks < kDv / 64) {
    if (conv == ks / 2) k8_convert<S>(r, d);
  }
  MLA_SB();
  if constexpr (S + kK8Ahead < N) k8_read<S + kK8Ahead>(ring[(S + kK8Ahead) % kK8Ring], a0, a1);
  MLA_SB();
  if constexpr (S + 1 == N) {
    mfma_tail();
  } else {
    constexpr int last = (S + kK8Ahead < N) ? S + kK8Ahead : N - 1;
    lgkm_wait<2 * (last - (S + 1))>();
  }
  MLA_SB();
  hook(ic<S>{});
  MLA_SB();
}

template <typename Hook, typename Pay, int... S>
__device__ __forceinline__ void s8_steps(f32x16& sc0, f32x16& sc1, K8 (&ring)[kK8Ring],
                                         const u32x8 (&qreg)[kKSteps8], uint32_t a0, uint32_t a1,
                                         const uint32_t (&d)[4], int conv, Hook& hook, Pay& pay,
                                         std::integer_sequence<int, S...>) {
  (s8_step<S>(sc0, sc1, ring, qreg, a0, a1, d, conv, hook, pay), ...);
}

template <int... S>
__device__ __forceinline__ void s8_prologue(K8 (&ring)[kK8Ring], uint32_t a0, uint32_t a1,
                                            std::integer_sequence<int, S...>) {
  (k8_read<S>(ring[S], a0, a1), ...);
}

// S^T of both key tiles of a page (sc0: keys 0..31, sc1: keys 32..63), 18
// MFMAs.  ka = LDS address of the lane's score operand in the page's
// staging buffer (see q8_offsets), d = its conversion addresses in the V
// page, conv = the wave's pair of column blocks.
template <typename Hook, typename Pay>
__device__ __forceinline__ void score_chain_q8(f32x16& sc0, f32x16& sc1,
                                               const u32x8 (&qreg)[kKSteps8], uint32_t ka,
                                               const uint32_t (&d)[4], int conv, Hook&& hook,
                                               Pay&& pay) {
  const uint32_t a1 = ka ^ 16u;
  K8 ring[kK8Ring];
  s8_prologue(ring, ka, a1, std::make_integer_sequence<int, kK8Ahead>{});
  lgkm_wait<2 * (kK8Ahead - 1)>();
  MLA_SB();
  s8_steps(sc0, sc1, ring, qreg, ka, a1, d, conv, hook, pay,
           std::make_integer_sequence<int, 2 * kKSteps8>{});
}

// Conversion share of a wave with no query rows (plain code): column blocks
// 2w and 2w + 1, all 64 keys, lane = key.
__device__ __forceinline__ void convert_share_q8(const uint8_t* stage, uint8_t* vpage, int wave) {
  const int key = (int)lane_id();
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int blk = 2 * wave + b;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + 4096 * blk + 64 * key +
                                                      16 * (c ^ f8_swz(key)));
      const u32x4 lo = cvt_chunk(v[0], v[1]), hi = cvt_chunk(v[2], v[3]);
      uint8_t* row = vpage + 8192 * blk + 128 * key;
      *reinterpret_cast<u32x4*>(row + 16 * ((2 * c) ^ chunk_swz(key))) = lo;
      *reinterpret_cast<u32x4*>(row + 16 * ((2 * c + 1) ^ chunk_swz(key))) = hi;
    }
  }
}

// Barrier for LDS data only: this wave's LDS operations are complete, then
// every wave meets.  (__syncthreads also waits for the wave's global loads,
// the next page's among them.)
__device__ __forceinline__ void lds_barrier() {
  lgkm_wait<0>();
  __builtin_amdgcn_s_barrier();
}

// Element placed in payload slot 8 + d when 16 elements are spread over 27
// slots (element i at 8 + 7i/4), or -1.
__host__ __device__ constexpr int spread_slot_elem(int d) {
  for (int i = 0; i < 16; ++i)
    if ((7 * i) / 4 == d) return i;
  return -1;
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

// FP8: the cache holds e4m3 bytes (kv_descale is read); else bf16.
// Q8 (with FP8): q holds e4m3 codes whose value is code * q_descale[0].
template <bool FP8, bool Q8>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_decode_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
                  const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
                  const int32_t* __restrict__ tile_plan, const int32_t* __restrict__ split_indptr,
                  const float* __restrict__ kv_descale, const float* __restrict__ q_descale,
                  uint16_t* __restrict__ partial_o, float* __restrict__ partial_lse,
                  uint16_t* __restrict__ out, float* __restrict__ lse_out, DecodeParams P) {
  static_assert(FP8 || !Q8, "an e4m3 query goes with an e4m3 cache");
  // bf16: two compute buffers.  fp8: compute buffer 0, and two e4m3 staging
  // buffers in the space of compute buffer 1.  fp8 query: the bf16 V page and
  // two staging buffers (see kQ8Stage).
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kPageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stage_all[kWaves][kStageBytes];
  constexpr int kSrcPageBytes = FP8 ? kPageBytesF8 : kPageBytes;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lane = (int)lane_id();  // used before the page loops only
  const int part = part_of_block(blockIdx.x, gridDim.x);

  const int32_t* tp = tile_plan + part * 8;
  const int b_first = tp[0], pg_first = tp[1], b_last = tp[2], pg_last = tp[3];
  const int first_piece = tp[4], total = tp[5];
  // An empty part, or a row no planner would produce, does nothing (the
  // check is uniform over the work-group, so no wave is left at a barrier).
  if (total <= 0 || b_first < 0 || b_last >= P.bs || b_first > b_last || pg_first < 0 ||
      first_piece < 0)
    return;

  const int row0 = blockIdx.y * kRowsPerBlock + wave * kRowsPerWave;  // first row of this wave
  const bool wave_active = row0 < P.rows;
  const int i_tok_min = row0 / P.heads;  // smallest token index among the wave's rows
  // This lane's query row is row0 + n, n = lane % 32.  That and the lane's
  // LDS offsets are recomputed where used, from a lane id read through pin()
  // (see lane_offsets), instead of being held across the page loop.

  // LDS starts as zeros: a load lane that falls outside a page's range may
  // leave its bytes untouched, and those bytes must be finite.
  for (int i = wave * 64 + lane; i < 2 * kPageBytes / 16; i += kWaves * 64)
    reinterpret_cast<u32x4*>(smem)[i] = (u32x4){0, 0, 0, 0};
  __syncthreads();

  // ---- page cursor for prefetch ----------------------------------------------
  // (nb, np) is the page whose loads are issued next.  Its block-table entry
  // (nraw) is read a whole page before it is used, and only checked when
  // used, so the scalar load never holds up the wave.
  int nb = b_first, np = pg_first;
  int nlen = uniform_load(seq_lens, nb);
  int nend = (nb == b_last) ? pg_last : page_count(nlen);
  auto raw_of = [&](int b, int p) -> int32_t {
    return p < P.bt_stride ? block_table[(int64_t)b * P.bt_stride + p] : -1;
  };
  int32_t nraw = raw_of(nb, np);
  // A block-table entry outside the pool (or a page past the table's width)
  // is a caller error: the page is not read (its loads get an empty range,
  // based at page 0) and every key of it is masked, so it contributes nothing.
  auto cursor_bad = [&]() -> uint32_t { return (nraw >= 0 && nraw < P.num_pages) ? 0u : 1u; };
  auto nphys = [&]() -> int64_t { return cursor_bad() ? 0 : nraw; };
  int nrows = min(kPage, max(0, nlen - np * kPage));
  // Loads of the cursor's page into LDS for page index `j` of the part.
  auto issue = [&](int j) {
    const int vr = __builtin_amdgcn_readfirstlane(cursor_bad() ? 0 : nrows);
    if constexpr (Q8)
      issue_loads_q8(std::make_integer_sequence<int, kKSteps8>{},
                     page_rsrc<kD>(kv + nphys() * kSrcPageBytes, vr),
                     smem + kQ8Stage + (j & 1) * kPageBytesF8, wave, q8_load_offset(lane, wave));
    else if constexpr (FP8)
      issue_loads_f8(std::make_integer_sequence<int, kLoadsPerWaveF8>{},
                     page_rsrc<kD>(kv + nphys() * kSrcPageBytes, vr),
                     smem + kPageBytes + (j & 1) * kPageBytesF8, wave, wave * 1024 + 16 * lane);
    else {
      const uint32_t lo = lane_offsets(lane, wave).load;
      issue_page_loads(page_rsrc<kRowBytes>(kv + nphys() * kSrcPageBytes, vr),
                       smem + (j & 1) * kPageBytes, wave, lo, lo + 4 * (8 * kRowBytes));
    }
  };
  // Move the cursor one page on and start reading that page's block-table
  // entry (a new request's length is needed at once, once per request).
  auto advance = [&]() {
    ++np;
    while (np >= nend && nb < b_last) {
      ++nb;
      np = 0;
      nlen = uniform_load(seq_lens, nb);
      nend = (nb == b_last) ? pg_last : page_count(nlen);
    }
    nraw = raw_of(nb, np);
    nrows = min(kPage, max(0, nlen - np * kPage));
  };

  issue(0);
  // bit 0: the page computed next is a bad one (see cursor_bad); bit 1: the
  // page after it
  uint32_t badq = cursor_bad();
  advance();

  // Every wave passes exactly `total` barriers, one per page, whatever the
  // plan says about requests, so a malformed plan cannot leave a wave
  // waiting at a barrier the others never reach.
  if (!wave_active) {
    // No query rows for this wave: it only helps stream the pages.
    for (int it = 0; it < total; ++it) {
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
      if (it + 1 < total) {
        issue(it + 1);
        advance();
      }
      if constexpr (Q8) {
        convert_share_q8(smem + kQ8Stage + (it & 1) * kPageBytesF8, smem, wave);
        lds_barrier();
      } else if constexpr (FP8) {
        convert_f8_page(smem + kPageBytes + (it & 1) * kPageBytesF8, smem, wave);
        __syncthreads();
      }
    }
    return;
  }

  // Range of the cursor's page for the loads issued during the page before
  // it.  It is worked out (and the cursor moved on, which starts the read of
  // the block-table entry after it) one page ahead, among the last output
  // MFMAs of a page, where the wave has issue slots to spare.
  // Returns whether the cursor's page is a bad one.
  __amdgpu_buffer_rsrc_t next_rsrc;
  auto next_range = [&](bool has) -> uint32_t {
    const uint32_t bad = has ? cursor_bad() : 0u;
    next_rsrc = page_rsrc<FP8 ? kD : kRowBytes>(
        kv + nphys() * kSrcPageBytes,
        (has && !bad) ? __builtin_amdgcn_readfirstlane(nrows) : 0);
    return bad;
  };
  badq |= next_range(1 < total) << 1;
  if (1 < total) advance();

  // Per-tensor dequantisation scale: scores use |delta| in the softmax scale
  // and the sign on q; the output is multiplied by delta.
  // An e4m3 query multiplies the scores by q_descale as well.
  const float delta = FP8 ? kv_descale[0] : 1.0f;
  const float qk_descale = Q8 ? delta * q_descale[0] : delta;
  // (kept above 0 so that a masked score, -inf, scales to -inf and never to
  // 0 * inf; a zero scale then weights the visible keys equally, to within
  // 1e-30 of a relative error)
  const float c_log2 = fmaxf(P.scale_log2 * fabsf(qk_descale), 1e-30f);
  const uint32_t q_sign =
      (FP8 && qk_descale < 0.f) ? (Q8 ? 0x80808080u : 0x80008000u) : 0u;

  // bf16 query: 36 k-steps of 8 values per lane; e4m3: 9 k-steps of 32.
  std::conditional_t<Q8, u32x8[kKSteps8], bf16x8[kKSteps]> qreg;
  f32x16 oacc[kVTiles];
  // Query rows of request b into qreg.  A lane whose row is past the last one
  // reads row 0 instead: its results stay in that lane's row of the
  // accumulators and are never stored, so no select on the loaded values
  // makes the wave wait for them where they are loaded.
  auto load_q = [&](int b) {
    const uint32_t ql = pinned_lane();
    const int r = row0 + (int)(ql & 31);
    if constexpr (Q8) {
      // lane (n, h): columns 64 ks + 32 h .. +31 of its row, the bytes the
      // score operand holds for the same lane
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(q) +
                            ((int64_t)b * P.rows + (r < P.rows ? r : 0)) * kD +
                            32 * (int)(ql >> 5);
#pragma unroll
      for (int ks = 0; ks < kKSteps8; ++ks) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(qrow + 64 * ks) ^ q_sign;
        const u32x4 hi = *reinterpret_cast<const u32x4*>(qrow + 64 * ks + 16) ^ q_sign;
        qreg[ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    } else {
      const uint16_t* qrow =
          q + ((int64_t)b * P.rows + (r < P.rows ? r : 0)) * kD + 8 * (int)(ql >> 5);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
        if (FP8) v ^= q_sign;
        qreg[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
  };
  int it = 0;  // pages of this part processed so far (selects the LDS buffer)
  int cb = b_first;
  int cp = pg_first;
  int piece = first_piece;
  // The queries of a piece after the first are loaded during the previous
  // piece's last page, once its last score MFMA has read them, and waited
  // for before that piece's output stores: vector memory operations complete
  // in order, so queries loaded after the stores would wait for them.
  bool first_wait = true;
  // Lane offsets and lane id into the first KiB of the wave's staging area
  // (again after each piece's output, which uses that area).
  // (fp8 query: the score operand and load offsets of its own layout)
  auto park_offsets = [&]() {
    const uint32_t pl = pinned_lane();
    const LaneOffsets o = lane_offsets(pl, wave);
    const uint32_t ok = Q8 ? q8_offsets(pl).k : o.k;
    const uint32_t ol = Q8 ? q8_load_offset(pl, wave) : o.load;
    *reinterpret_cast<u32x4*>(stage_all[wave] + 16 * pl) = (u32x4){ok, o.v, ol, pl};
  };
  park_offsets();
  load_q(cb);
  // the first page and the queries land here, so that no path into the page
  // loop below leaves query loads in flight (the compiler would otherwise
  // wait for them at the score MFMAs of every page, behind the next page's
  // loads issued there)
  __builtin_amdgcn_s_waitcnt(0x0f70);
  while (true) {
    // ---- one piece: pages [cp, cend) of request cb ---------------------------
    const int32_t L = uniform_load(seq_lens, cb);
    const int cend = (cb == b_last) ? pg_last : page_count(L);
    // pages from first_masked on may hold keys some row of this wave cannot see
    const int32_t lim_min = P.causal ? L - P.q_len + i_tok_min : L - 1;
    const int first_masked =
        __builtin_amdgcn_readfirstlane(lim_min >= 0 ? (lim_min + 1) / kPage : 0);
    // the part's next request that has pages (if the part goes on past this one)
    int ncb = cb;
    if (cb < b_last) {
      do {
        ++ncb;
      } while (ncb < b_last && page_count(uniform_load(seq_lens, ncb)) <= 0);
    }
    // on the piece's last page, if another piece follows: load its queries
    // and wait for them at once (with the load in the same branch, no path
    // back to the score MFMAs leaves query loads in flight; the compiler
    // would otherwise wait for them at the score MFMAs of every page, behind
    // the next page's loads issued there)
    auto prefetch_q = [&]() {
      if (cp + 1 == cend && it + 1 < total && cb < b_last) {
        load_q(ncb);
        __builtin_amdgcn_s_waitcnt(0x0f70);
      }
    };
    zero_acc(oacc);
    float m_run = -INFINITY, l_run = 0.f;

    // One page of the piece.  MASKED: some key of the page may be invisible to
    // some row of the wave (page tail, causal limit); on those pages (at most
    // the last one or, for several tokens per request, the last few) the
    // scores of such keys are masked before the softmax.  The two kinds are
    // two instances of the same code, run as two loops.
    auto page = [&](auto masked_c) {
      constexpr bool MASKED = decltype(masked_c)::value;
      // vmcnt(0): this wave's loads of page `it` landed (for a piece's first
      // page after the first piece: waited for before the previous epilogue);
      // the barrier: every wave's, and buffer it+1 is free again
      // this lane's LDS offsets and id, kept in the wave's staging area: read
      // before the barrier, so that the read's latency overlaps the wait
      const u32x4 lov = *reinterpret_cast<const u32x4*>(stage_all[wave] + 16 * lane_id());
      if (first_wait) __builtin_amdgcn_s_waitcnt(0x0f70);
      first_wait = true;
      __syncthreads();
      const uint32_t plane = lov[3];
      const LaneOffsets lo = {lov[0], lov[1], lov[2]};
      const bool bad = badq & 1u;  // uniform: this page is a bad one, mask all its keys
      // the page's LDS buffer: the compute page (fp8 query: the e4m3 staging
      // buffer, which the score operands are read from)
      const lds_u8* base =
          LDS_PTR(uint8_t, smem) +
          (Q8 ? kQ8Stage + (it & 1) * kPageBytesF8 : FP8 ? 0 : (it & 1) * kPageBytes);
      // The next page's loads are spread over the MFMA work (issued back to
      // back they would stall the wave until the address unit drains them).
      // Their range (next_rsrc) was worked out on the previous page.  After the
      // part's last page the loads still go out, over an empty range: they
      // only write zeros into the free buffer (and cost no branch per load);
      // the kernel waits for them before it ends.
      uint8_t* const next_buf = Q8    ? smem + kQ8Stage + ((it + 1) & 1) * kPageBytesF8
                                : FP8 ? smem + kPageBytes + ((it + 1) & 1) * kPageBytesF8
                                      : smem + ((it + 1) & 1) * kPageBytes;
      // load K of this wave's share, K < 18 (bf16) or K < 9 (e4m3)
      auto load = [&](auto kc) {
        constexpr int K = decltype(kc)::value;
        if constexpr (Q8)
          issue_one_load_q8<K>(next_rsrc, next_buf, wave, lo.load);
        else if constexpr (FP8)
          issue_one_load_f8<K>(next_rsrc, next_buf, wave, wave * 1024 + 16 * plane);
        else
          issue_one_load<K>(next_rsrc, next_buf, wave, lo.load, lo.load + 4 * (8 * kRowBytes));
      };
      auto hook_s0 = [&](auto g) { load(g); };
      auto no_hook = [](auto) {};
      if constexpr (FP8 && !Q8) {
        convert_f8_page(smem + kPageBytes + (it & 1) * kPageBytesF8, smem, wave);
        __syncthreads();  // the compute page is complete
      }

      // LDS byte addresses of this page's operands (fp8 query: V from the
      // bf16 V page at the start of the LDS buffers)
      const uint32_t pbase = (uint32_t)(uintptr_t)base;
      const uint32_t vbase = Q8 ? (uint32_t)(uintptr_t)LDS_PTR(uint8_t, smem) : pbase;
      const uint32_t ka = pbase + lo.k, va = vbase + lo.v;

      {
        // The softmax of each tile runs in the shadow of the matrix work:
        //   S(0)
        //   S(1) + PV(0) mixed | max(0), rescale decision, weights P(0);
        //                        then max(1) and P(1) for keys 0..15 of the tile,
        //                        under the running max as it stands
        //   (rare: the running max moves for tile 1 -> rescale, redo those weights)
        //   PV(1) | weights P(1) for keys 16..31 (used from group 4 on)
        // sc0[i] / sc1[i] is key 16h + i of tile 0 / 1.  On a MASKED page the
        // scores of keys a row cannot see are set to -inf before the row max
        // (weights 2^-inf = 0).
        f32x16 sc0, sc1;
        int vis0 = 16, vis1 = 16;  // elements i < vis of the lane's 16 are visible keys
        if constexpr (MASKED) {
          const int r = row0 + (int)(plane & 31);
          const int i_tok = r < P.rows ? r / P.heads : 0;
          const int32_t lim = P.causal ? L - P.q_len + i_tok : L - 1;  // last visible key
          vis0 = bad ? 0 : lim - (cp * kPage + 16 * (int)(plane >> 5)) + 1;
          vis1 = vis0 - 32;
        }
        auto mask_tile = [&](f32x16& sc, int vis) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[i] = i < vis ? sc[i] : -INFINITY;
        };
        // the masking of tile sc: by vis on a MASKED page; on another page
        // only if the page is a bad one (a uniform branch)
        auto mask = [&](f32x16& sc, int vis) {
          if constexpr (MASKED) {
            mask_tile(sc, vis);
          } else if (bad) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[i] = -INFINITY;
          }
        };

        float mx[4], ls[4];
        float m_tile = 0.f, neg_m = 0.f;
        bool need = false;
        uint32_t pk[8];
        // row max of tile `sc`, part k (k < 4: 4 of the 16 values; k == 4: the
        // rest): m_tile
        auto max_part = [&](const f32x16& sc, auto part) {
          constexpr int k = decltype(part)::value;
          if constexpr (k < 4) {
            mx[k] = fmaxf(fmaxf(sc[k], sc[k + 4]), fmaxf(sc[k + 8], sc[k + 12]));
            keep(mx[k]);
          } else {
            const float mloc = xhalf_max(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])));
            m_tile = c_log2 * mloc;
            keep(m_tile);
          }
        };
        // weights of elements i, i + 1 of tile `sc` (i even), packed to bf16 in
        // pk[i / 2]; their sum goes to ls
        auto weight2 = [&](const f32x16& sc, auto ii) {
          constexpr int i = decltype(ii)::value;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[i], c_log2, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[i + 1], c_log2, neg_m));
          ls[i & 3] += p0;
          ls[(i + 1) & 3] += p1;
          keep(ls[i & 3]), keep(ls[(i + 1) & 3]);
          pk[i >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0, p1}, bf16x2));
          keep(pk[i >> 1]);
        };
        auto fold_ls = [&]() {
          l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
          keep(l_run);
#pragma unroll
          for (int j = 0; j < 4; ++j) ls[j] = 0.f;
        };
        // lazy rescale: move the running max only when the tile's max exceeds it by
        // more than kTau (p <= 2^kTau otherwise); rows still at -inf have o = 0.
        // Call only with no output MFMA in flight.
        auto rescale = [&]() {
          const float m_new = need ? m_tile : m_run;
          const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
          l_run *= alpha;
          if (__any(need && m_run != -INFINITY)) {
#pragma unroll
            for (int vt = 0; vt < kVTiles; ++vt) scale_tile(oacc[vt], alpha);
          }
          m_run = m_new;
          neg_m = m_run == -INFINITY ? 0.f : -m_run;  // -inf: no visible key yet
        };
        bf16x8 pop[2];
        // weights of keys 16..31 in slots 1, 5, 9, 13 (used from MFMA 16 on)
        auto pay_pv1 = [&](auto slot) {
          constexpr int k = decltype(slot)::value;
          if constexpr (k < 16 && k % 4 == 1) {
            weight2(sc1, ic<(k - 1) / 2 + 8>{});
            if constexpr (k == 13)
              pop[1] = __builtin_bit_cast(bf16x8, (u32x4){pk[4], pk[5], pk[6], pk[7]});
          } else if constexpr (k == 14) {
            fold_ls();
          } else if constexpr (k == 17) {
            // page it + 2, loaded during page it + 1
            badq = (badq >> 1) | (next_range(it + 2 < total) << 1);
          } else if constexpr (k == 21) {
            if (it + 2 < total) advance();
          }
        };
        // the running max moves for tile 1 (the output chain of tile 0 has
        // drained): rescale, and redo the weights of keys 0..7 under the new max
        auto redo_tile1 = [&]() {
          if (__any(need)) {
            rescale();
#pragma unroll
            for (int j = 0; j < 4; ++j) ls[j] = 0.f;
            weight2(sc1, ic<0>{});
            weight2(sc1, ic<2>{});
            weight2(sc1, ic<4>{});
            weight2(sc1, ic<6>{});
          }
          pop[0] = __builtin_bit_cast(bf16x8, (u32x4){pk[0], pk[1], pk[2], pk[3]});
        };
        if constexpr (Q8) {
          // fp8 query:
          //   S(0), S(1) as one chain of 18 | the next page's loads (steps 0..8),
          //     this wave's V conversion, max(0), rescale decision, P(0) keys 0..7
          //   barrier: every wave's share of the V page is written
          //   PV(0) | P(0) keys 8..15, max(1), P(1) keys 0..7 under the running max
          //   (rare: the running max moves for tile 1 -> rescale, redo those weights)
          //   PV(1) | P(1) keys 8..15
          const uint32_t d0 = vbase + q8_offsets(plane).d;
          const uint32_t dq[4] = {d0, d0 ^ 16u, d0 ^ 32u, d0 ^ 48u};
          auto hook_s8 = [&](auto step) {
            constexpr int k = decltype(step)::value;
            if constexpr (k < kKSteps8) {
              load(step);
            } else if constexpr (k == kKSteps8 + 4) {
              need = m_tile > m_run + kTau;
              if (__any(need)) rescale();
              neg_m = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
              for (int j = 0; j < 4; ++j) ls[j] = 0.f;
            }
          };
          auto pay_s8 = [&](auto step) {
            constexpr int k = decltype(step)::value - kKSteps8;  // step of tile 1
            if constexpr (k == 0) {
              // the last MFMA of tile 0 went out one step before: let it land
              asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
              MLA_SB();  // (reads of sc0 stay below the wait states)
              mask(sc0, vis0);
            }
            if constexpr (k >= 0 && k < 5) {
              max_part(sc0, ic<k>{});
            } else if constexpr (k >= 5) {
              weight2(sc0, ic<2 * (k - 5)>{});
              if constexpr (k == 8)
                pop[0] = __builtin_bit_cast(bf16x8, (u32x4){pk[0], pk[1], pk[2], pk[3]});
            }
          };
          score_chain_q8(sc0, sc1, qreg, ka, dq, wave, hook_s8, pay_s8);
          prefetch_q();
          lds_barrier();
          auto pay_pv0 = [&](auto slot) {
            constexpr int k = decltype(slot)::value;
            if constexpr (k < 8 && k % 2 == 1) {
              weight2(sc0, ic<k + 7>{});  // elements 8, 10, 12, 14
              if constexpr (k == 7)
                pop[1] = __builtin_bit_cast(bf16x8, (u32x4){pk[4], pk[5], pk[6], pk[7]});
            } else if constexpr (k == 8) {
              fold_ls();
            } else if constexpr (k >= 10 && k < 15) {
              if constexpr (k == 10) mask(sc1, vis1);
              max_part(sc1, ic<k - 10>{});
            } else if constexpr (k >= 16 && k < 24 && k % 2 == 0) {
              weight2(sc1, ic<k - 16>{});
            }
          };
          auto hook_pv0 = [&](auto group) {
            if constexpr (decltype(group)::value == 3) need = m_tile > m_run + kTau;
          };
          pv_tile<0>(oacc, pop, va, hook_pv0, pay_pv0);
          redo_tile1();
          pv_tile<1>(oacc, pop, va, no_hook, pay_pv1);
        } else {
          score_tile<0>(sc0, ka, qreg, hook_s0, NoSlot{});
          // payload slots of the combined chain
          constexpr int kE0 = 5;                 // tile 0, keys 0..7: slots 5..8
          constexpr int kE1 = kCPrefix + 1;      // tile 0, keys 8..15: slots 10, 16, 22, 28
          constexpr int kLd = kCPrefix + 2;      // bf16 loads 9..17: slots 11, 14, .., 35
          constexpr int kM1 = kCLastScore + 1;   // max(1): slots 59..63
          constexpr int kW1 = kM1 + 5;           // tile 1, keys 0..7: slots 64..67
          static_assert(kE0 + 4 == kCPrefix && kCPrefix == kCFirstOut && kE1 + 6 * 3 < kCOutU1 &&
                            kW1 + 4 == kCSlots,
                        "combined chain payload layout");
          auto pay_c = [&](auto slot) {
            constexpr int k = decltype(slot)::value;
            if constexpr (k < kE0) {
              if constexpr (k == 0) mask(sc0, vis0);
              max_part(sc0, slot);
            } else if constexpr (k < kE0 + 4) {
              weight2(sc0, ic<2 * (k - kE0)>{});
              if constexpr (k == kE0 + 3)
                pop[0] = __builtin_bit_cast(bf16x8, (u32x4){pk[0], pk[1], pk[2], pk[3]});
            } else if constexpr (k >= kE1 && k <= kE1 + 6 * 3 && (k - kE1) % 6 == 0) {
              weight2(sc0, ic<8 + 2 * ((k - kE1) / 6)>{});
              if constexpr (k == kE1 + 6 * 3) {
                pop[1] = __builtin_bit_cast(bf16x8, (u32x4){pk[4], pk[5], pk[6], pk[7]});
                fold_ls();
              }
            } else if constexpr (k >= kM1 && k < kM1 + 5) {
              // the last score MFMA went out one slot before: let its result land
              if constexpr (k == kM1) {
                asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
                MLA_SB();  // (reads of sc1 stay below the wait states)
                mask(sc1, vis1);
              }
              max_part(sc1, ic<k - kM1>{});
            } else if constexpr (k >= kW1) {
              weight2(sc1, ic<2 * (k - kW1)>{});
            }
          };
          auto hook_c = [&](auto slot) {
            constexpr int k = decltype(slot)::value;
            if constexpr (k == kE0 - 1) {
              need = m_tile > m_run + kTau;
              if (__any(need)) rescale();
              neg_m = m_run == -INFINITY ? 0.f : -m_run;
  #pragma unroll
              for (int j = 0; j < 4; ++j) ls[j] = 0.f;
            } else if constexpr (k == kW1 - 1) {
              need = m_tile > m_run + kTau;
            } else if constexpr (!FP8 && k >= kLd && k <= kLd + 3 * 8 && (k - kLd) % 3 == 0) {
              load(ic<9 + (k - kLd) / 3>{});
            }
          };
          combined_chain(sc1, oacc, pop, qreg, ka, va, hook_c, pay_c);
          prefetch_q();
          redo_tile1();
          pv_tile<1>(oacc, pop, va, no_hook, pay_pv1);
        }
      }
    };

    const int cfast = min(cend, max(cp, first_masked));
    for (; cp < cfast && it < total; ++cp, ++it) page(std::false_type{});
    for (; cp < cend && it < total; ++cp, ++it) page(std::true_type{});

    // ---- epilogue of the piece ---------------------------------------------------
    const bool more = it < total && cb < b_last;
    if (more) {
      // the next piece's queries and first page land before any store goes out
      __builtin_amdgcn_s_waitcnt(0x0f70);
      first_wait = false;
    }
    {
      const float l_tot = xhalf_sum(l_run);
      const float inv = l_tot > 0.f ? delta / l_tot : 0.f;
      const float lse_val =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
      const int k0 = uniform_load(split_indptr, cb);
      const int k = uniform_load(split_indptr, cb + 1) - k0;
      const int64_t slot = (int64_t)k0 + piece;
      // A piece of a split request goes to its partial slot (normalised o and
      // lse, fp32); the only piece of a request is final (bf16 o).
      const bool to_partial = k > 1;
      const uint32_t ln = pinned_lane();
      const int r = row0 + (int)(ln & 31);
      if (to_partial && slot >= 0 && slot < P.partial_slots) {
        if ((ln >> 5) == 0 && r < P.rows) partial_lse[slot * P.rows + r] = lse_val;
        uint16_t* const po = partial_o + slot * P.rows * kDv;
        if (row0 + kRowsPerWave <= P.rows)
          store_rows<uint16_t, true>(oacc, inv, stage_all[wave], po, row0, P.rows, ln);
        else
          store_rows<uint16_t, false>(oacc, inv, stage_all[wave], po, row0, P.rows, ln);
      } else if (!to_partial) {
        if (lse_out && (ln >> 5) == 0 && r < P.rows) lse_out[(int64_t)cb * P.rows + r] = lse_val;
        uint16_t* const ob = out + (int64_t)cb * P.rows * kDv;
        if (row0 + kRowsPerWave <= P.rows)
          store_rows<uint16_t, true>(oacc, inv, stage_all[wave], ob, row0, P.rows, ln);
        else
          store_rows<uint16_t, false>(oacc, inv, stage_all[wave], ob, row0, P.rows, ln);
      }
    }
    if (!more) break;
    park_offsets();
    cb = ncb;
    cp = 0;
    piece = 0;
  }
  // Only reached early with a malformed plan: keep the barrier count.
  for (; it < total; ++it) {
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if constexpr (FP8) __syncthreads();
  }
  // the last page's empty loads land before the work-group's LDS is released
  __builtin_amdgcn_s_waitcnt(0x0f70);
}

}  // namespace mla

namespace {
// Events for the next launch on this thread (mla_decode_time_next_launch).
thread_local hipEvent_t t_start_event = nullptr, t_stop_event = nullptr;
}  // namespace

extern "C" mla_status mla_decode_time_next_launch(hipEvent_t start, hipEvent_t stop) {
  t_start_event = start;
  t_stop_event = stop;
  return mla::ok();
}

namespace mla {
namespace {

// mla_decode and mla_decode_q8: checks, then the launch.  q8: q holds e4m3
// codes scaled by *q_descale, over an e4m3 cache.
mla_status decode_impl(const char* name, const void* q, const float* q_descale, bool q8,
                       int32_t bs, int32_t q_len, int32_t num_heads, const void* kv_cache,
                       int32_t kv_dtype, int64_t num_pages, const int32_t* block_table,
                       int32_t bt_row_stride, const int32_t* seq_lens, const int32_t* tile_plan,
                       int32_t num_parts, const int32_t* split_indptr, float softmax_scale,
                       int32_t causal, const float* kv_descale, void* partial_o,
                       float* partial_lse, int32_t partial_slots, void* out, float* lse,
                       hipStream_t stream) {
  const std::string n(name);
  const hipEvent_t ev_start = t_start_event, ev_stop = t_stop_event;
  t_start_event = t_stop_event = nullptr;
  if (!q || !kv_cache || !block_table || !seq_lens || !tile_plan || !split_indptr || !partial_o ||
      !partial_lse || !out || (q8 && !q_descale))
    return fail(MLA_ERR_INVALID_ARGUMENT, n + ": null pointer");
  if (bs <= 0 || q_len <= 0 || num_heads <= 0 || num_pages <= 0 || bt_row_stride <= 0 ||
      num_parts <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, n + ": sizes must be positive");
  if (!finite_nonneg(softmax_scale))
    return fail(MLA_ERR_INVALID_ARGUMENT, n + ": softmax_scale must be finite and >= 0");
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, n + ": unknown kv_dtype");
  if (q8 && kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, n + ": an e4m3 query needs an e4m3 cache");
  if (kv_dtype == MLA_KV_FP8_E4M3 && !kv_descale)
    return fail(MLA_ERR_INVALID_ARGUMENT, n + ": fp8 cache needs kv_descale");
  const int64_t rows = (int64_t)q_len * num_heads;
  if (rows < 1 || rows > MLA_MAX_ROWS_PER_REQ)
    return fail(MLA_ERR_UNSUPPORTED, n + ": q_len*num_heads must be in 1..512");
  if (num_parts > MLA_MAX_DECODE_PARTS)
    return fail(MLA_ERR_CAPACITY, n + ": num_parts above " + std::to_string(MLA_MAX_DECODE_PARTS));
  if ((int64_t)bs * bt_row_stride >= (int64_t)1 << 29)
    return fail(MLA_ERR_UNSUPPORTED, n + ": the block table must hold fewer than 2^29 entries");
  if ((int64_t)partial_slots < (int64_t)bs + num_parts)
    return fail(MLA_ERR_CAPACITY, n + ": partial_slots must be at least bs + num_parts");

  DecodeParams p;
  p.num_pages = num_pages;
  p.partial_slots = partial_slots;
  p.bt_stride = bt_row_stride;
  p.bs = bs;
  p.q_len = q_len;
  p.heads = num_heads;
  p.rows = (int32_t)rows;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  dim3 grid(num_parts, (unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
#ifdef MLA_DEBUG
  {
    const mla_status checked = debug_check_table_entries(name, block_table, bt_row_stride,
                                                         seq_lens, bs, num_pages, stream);
    if (checked != MLA_OK) return checked;
  }
#endif
  trace("%s: bs %d q_len %d heads %d kv_dtype %d%s pages %lld width %d parts %d slots %d "
        "grid %ux%u stream %p",
        name, bs, q_len, num_heads, kv_dtype, q8 ? " (e4m3 query)" : "", (long long)num_pages,
        bt_row_stride, num_parts, partial_slots, grid.x, grid.y, (void*)stream);
  auto launch = [&](auto kernel) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(q);
    const uint8_t* kvp = reinterpret_cast<const uint8_t*>(kv_cache);
    const float* kd = kv_dtype == MLA_KV_FP8_E4M3 ? kv_descale : nullptr;
    const float* qd = q8 ? q_descale : nullptr;
    uint16_t* op = reinterpret_cast<uint16_t*>(out);
    uint16_t* po = reinterpret_cast<uint16_t*>(partial_o);
    if (ev_start || ev_stop)
      hipExtLaunchKernelGGL(kernel, grid, dim3(kWaves * 64), 0, stream, ev_start, ev_stop, 0, qp,
                            kvp, block_table, seq_lens, tile_plan, split_indptr, kd, qd, po,
                            partial_lse, op, lse, p);
    else
      hipLaunchKernelGGL(kernel, grid, dim3(kWaves * 64), 0, stream, qp, kvp, block_table,
                         seq_lens, tile_plan, split_indptr, kd, qd, po, partial_lse, op, lse, p);
  };
  if (q8)
    launch(mla_decode_kernel<true, true>);
  else if (kv_dtype == MLA_KV_FP8_E4M3)
    launch(mla_decode_kernel<true, false>);
  else
    launch(mla_decode_kernel<false, false>);
  return check_launch(name);
}

}  // namespace
}  // namespace mla

extern "C" mla_status mla_decode(const void* q, int32_t bs, int32_t q_len, int32_t num_heads,
                                 const void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                                 const int32_t* block_table, int32_t bt_row_stride,
                                 const int32_t* seq_lens, const int32_t* tile_plan,
                                 int32_t num_parts, const int32_t* split_indptr,
                                 float softmax_scale, int32_t causal, const float* kv_descale,
                                 void* partial_o, float* partial_lse, int32_t partial_slots,
                                 void* out, float* lse, hipStream_t stream) {
  return mla::decode_impl("mla_decode", q, nullptr, false, bs, q_len, num_heads, kv_cache,
                          kv_dtype, num_pages, block_table, bt_row_stride, seq_lens, tile_plan,
                          num_parts, split_indptr, softmax_scale, causal, kv_descale, partial_o,
                          partial_lse, partial_slots, out, lse, stream);
}

extern "C" mla_status mla_decode_q8(const void* q_fp8, const float* q_descale, int32_t bs,
                                    int32_t q_len, int32_t num_heads, const void* kv_cache,
                                    int64_t num_pages, const int32_t* block_table,
                                    int32_t bt_row_stride, const int32_t* seq_lens,
                                    const int32_t* tile_plan, int32_t num_parts,
                                    const int32_t* split_indptr, float softmax_scale,
                                    int32_t causal, const float* kv_descale, void* partial_o,
                                    float* partial_lse, int32_t partial_slots, void* out,
                                    float* lse, hipStream_t stream) {
  return mla::decode_impl("mla_decode_q8", q_fp8, q_descale, true, bs, q_len, num_heads,
                          kv_cache, MLA_KV_FP8_E4M3, num_pages, block_table, bt_row_stride,
                          seq_lens, tile_plan, num_parts, split_indptr, softmax_scale, causal,
                          kv_descale, partial_o, partial_lse, partial_slots, out, lse, stream);
}
