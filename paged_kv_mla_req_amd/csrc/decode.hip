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
constexpr float kTau = 8.0f;
// The page loop issues the next page's loads one per MFMA block: after the 9
// score blocks and 8 output blocks of the first tile, and the first score
// block of the second (bf16: 18 loads; e4m3: 9, all in the first score tile).
static_assert(kLoadsPerWave == 18 && kLoadsPerWaveF8 == 9 && kKSteps / 4 == 9,
              "load spreading assumes 18 / 9 loads and 9 score blocks");                             // lazy-rescale threshold (log2 units)

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
                                           (K & 1) ? voff1 : voff0, 0, imm, 0);
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

// e4m3 page: a plain copy into a 36 KiB staging buffer.  Load k of wave w
// fills staging bytes [1024 j, 1024 j + 1024) with j = w + 4k from the same
// page offsets; voff = 1024 w + 16 lane.
template <int... K>
__device__ __forceinline__ void issue_loads_f8(std::integer_sequence<int, K...>,
                                               __amdgpu_buffer_rsrc_t rsrc, uint8_t* stage,
                                               int wave, uint32_t voff) {
  (__builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc,
                                            LDS_PTR(void, stage + 1024 * (wave + kWaves * K)),
                                            16, voff + 4096 * K, 0, 0, 0),
   ...);
}

template <int K>
__device__ __forceinline__ void issue_one_load_f8(__amdgpu_buffer_rsrc_t rsrc, uint8_t* stage,
                                                  int wave, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, stage + 1024 * (wave + kWaves * K)),
                                           16, voff + 4096 * K, 0, 0, 0);
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
__device__ __forceinline__ void convert_f8_page(const uint8_t* stage, uint8_t* buf) {
  const int key = threadIdx.x >> 2;
  const int c0 = 2 * (threadIdx.x & 3);
  const int slot0 = c0 ^ chunk_swz(key);
  const uint8_t* src = stage + key * kD + 16 * (threadIdx.x & 3);
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
// The two MFMA chains of a page are issued from inline assembly in blocks of
// four MFMAs.  Each block first issues the LDS reads of the *next* block's
// operands, then its own MFMAs, then waits for those reads: the reads are
// always in flight behind 128 cycles of matrix work, and no register leaves
// a block with a load still pending, so the compiler may move or copy any
// block output freely.  (Left to itself the compiler sinks every read next
// to its MFMA, because the kernel sits at the 512-register limit.)
// Hazards the compiler cannot see are covered by hand: 2 wait states before
// the MFMAs of a block (a VALU write of an operand just before), and 24
// after the last MFMA of a chain (MFMA result -> VALU / accumulator read;
// more than the 18 a 16-pass MFMA needs).
// ---------------------------------------------------------------------------

// S^T block: reads K operands at a[i] + OFF into nk, then 4 MFMAs on k.
template <int OFF>
__device__ __forceinline__ void s_block(f32x16& sc, bf16x8 (&nk)[4], const bf16x8 (&k)[4],
                                        const bf16x8* q, const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b128 %1, %13 offset:%17\n\t"
      "ds_read_b128 %2, %14 offset:%17\n\t"
      "ds_read_b128 %3, %15 offset:%17\n\t"
      "ds_read_b128 %4, %16 offset:%17\n\t"
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %9, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %6, %10, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %7, %11, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %8, %12, %0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "+v"(sc), "=&v"(nk[0]), "=&v"(nk[1]), "=&v"(nk[2]), "=&v"(nk[3])
      : "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]),
        "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF));
}

// First S^T block of a tile: the accumulator starts from 0.
template <int OFF>
__device__ __forceinline__ void s_block_first(f32x16& sc, bf16x8 (&nk)[4], const bf16x8 (&k)[4],
                                              const bf16x8* q, const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b128 %1, %13 offset:%17\n\t"
      "ds_read_b128 %2, %14 offset:%17\n\t"
      "ds_read_b128 %3, %15 offset:%17\n\t"
      "ds_read_b128 %4, %16 offset:%17\n\t"
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %9, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %6, %10, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %7, %11, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %8, %12, %0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(sc), "=&v"(nk[0]), "=&v"(nk[1]), "=&v"(nk[2]), "=&v"(nk[3])
      : "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]),
        "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF));
}

// Last S^T block: no further reads; the result is read by VALU next.
__device__ __forceinline__ void s_block_last(f32x16& sc, const bf16x8 (&k)[4], const bf16x8* q) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %5, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %6, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %7, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %8, %0\n\t"
      "s_nop 7\n\t"
      "s_nop 7\n\t"
      "s_nop 7"
      : "+v"(sc)
      : "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]));
}

// a[i] for column blocks >= 8: the DS offset field stops at 65535.
template <int G, int TB>
__device__ __forceinline__ void s_step(f32x16& sc, bf16x8 (&kk)[2][4], const bf16x8 (&qreg)[kKSteps],
                                       const uint32_t (&a)[4], const uint32_t (&a_hi)[4]) {
  constexpr int NOFF = 8192 * (G + 1) + TB;  // byte offset of the next group's reads
  if constexpr (G == 0)
    s_block_first<NOFF>(sc, kk[1], kk[0], &qreg[0], a);
  else if constexpr (G + 1 < kKSteps / 4) {
    if constexpr (NOFF < 65536)
      s_block<NOFF>(sc, kk[(G + 1) & 1], kk[G & 1], &qreg[4 * G], a);
    else
      s_block<NOFF - 32768>(sc, kk[(G + 1) & 1], kk[G & 1], &qreg[4 * G], a_hi);
  } else {
    s_block_last(sc, kk[G & 1], &qreg[4 * G]);
  }
}

template <int TB, typename Hook, int... G>
__device__ __forceinline__ void s_chain(f32x16& sc, bf16x8 (&kk)[2][4],
                                        const bf16x8 (&qreg)[kKSteps], const uint32_t (&a)[4],
                                        const uint32_t (&a_hi)[4], Hook& hook,
                                        std::integer_sequence<int, G...>) {
  ((s_step<G, TB>(sc, kk, qreg, a, a_hi), hook(std::integral_constant<int, G>{})), ...);
}

// S^T for the 32-key tile at byte offset TB of the page: 36 MFMAs in 9
// blocks; hook(integral_constant<G>) runs after block G (the page loop uses
// it to spread the next page's global loads over the matrix work).
// a[i] = page + koff[i] (LDS byte addresses), a_hi[i] = a[i] + 32768.
template <int TB, typename Hook>
__device__ __forceinline__ void score_tile(f32x16& sc, const uint32_t (&a)[4],
                                           const uint32_t (&a_hi)[4],
                                           const bf16x8 (&qreg)[kKSteps], Hook&& hook) {
  bf16x8 kk[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    kk[0][i] = *LDS_PTR(const bf16x8, (uintptr_t)(a[i] + TB));
  s_chain<TB>(sc, kk, qreg, a, a_hi, hook, std::make_integer_sequence<int, kKSteps / 4>{});
}

// PV blocks run four MFMAs each (one accumulator tile per MFMA) from a ring
// of three operand sets: block b computes with set b % 3 and issues the reads
// of block b + 2 into set (b + 2) % 3, then waits until at most those eight
// reads are outstanding, i.e. until block b + 1's operands have landed.  The
// reads of a block therefore have two blocks (256 cycles) of matrix work to
// arrive.  Set (b + 2) % 3 is an output of block b but is first read by
// block b + 2, after block b + 1 has waited for it.
// V^T operand reads of one MFMA: two transposing 8-byte reads (keys
// kb..kb+3 and kb+4..kb+7) at va[0][par] + off and va[1][par] + off.
#define MLA_PV_READS                                   \
  "ds_read_b64_tr_b16 %4, %17 offset:%21\n\t"          \
  "ds_read_b64_tr_b16 %8, %18 offset:%21\n\t"          \
  "ds_read_b64_tr_b16 %5, %19 offset:%21\n\t"          \
  "ds_read_b64_tr_b16 %9, %20 offset:%21\n\t"          \
  "ds_read_b64_tr_b16 %6, %17 offset:%22\n\t"          \
  "ds_read_b64_tr_b16 %10, %18 offset:%22\n\t"         \
  "ds_read_b64_tr_b16 %7, %19 offset:%22\n\t"          \
  "ds_read_b64_tr_b16 %11, %20 offset:%22\n\t"

// Block with reads ahead.  WAIT is the number of LDS reads allowed to stay
// outstanding at the end (8: the ones just issued).
template <int OFF0, int OFF1, int WAIT>
__device__ __forceinline__ void pv_block_rd(f32x16& o0, f32x16& o1, f32x16& o2, f32x16& o3,
                                            bf16x4 (&nlo)[4], bf16x4 (&nhi)[4],
                                            const bf16x8 (&v)[4], bf16x8 p,
                                            const uint32_t (&va)[2][2]) {
  asm volatile(
      MLA_PV_READS
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %12, %16, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %13, %16, %1\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %14, %16, %2\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %15, %16, %3\n\t"
      "s_waitcnt lgkmcnt(%23)"
      : "+a"(o0), "+a"(o1), "+a"(o2), "+a"(o3), "=&v"(nlo[0]), "=&v"(nlo[1]), "=&v"(nlo[2]),
        "=&v"(nlo[3]), "=&v"(nhi[0]), "=&v"(nhi[1]), "=&v"(nhi[2]), "=&v"(nhi[3])
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(p), "v"(va[0][0]), "v"(va[1][0]),
        "v"(va[0][1]), "v"(va[1][1]), "i"(OFF0), "i"(OFF1), "i"(WAIT));
}

// Block without reads; WAIT as above (0: drain), LAST adds the tail that
// lets VALU read the accumulators next.
template <int WAIT, bool LAST>
__device__ __forceinline__ void pv_block_nord(f32x16& o0, f32x16& o1, f32x16& o2, f32x16& o3,
                                              const bf16x8 (&v)[4], bf16x8 p) {
  if constexpr (LAST)
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %8, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %5, %8, %1\n\t"
        "v_mfma_f32_32x32x16_bf16 %2, %6, %8, %2\n\t"
        "v_mfma_f32_32x32x16_bf16 %3, %7, %8, %3\n\t"
        "s_nop 7\n\t"
        "s_nop 7\n\t"
        "s_nop 7"
        : "+a"(o0), "+a"(o1), "+a"(o2), "+a"(o3)
        : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(p));
  else
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %8, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %5, %8, %1\n\t"
        "v_mfma_f32_32x32x16_bf16 %2, %6, %8, %2\n\t"
        "v_mfma_f32_32x32x16_bf16 %3, %7, %8, %3\n\t"
        "s_waitcnt lgkmcnt(%9)"
        : "+a"(o0), "+a"(o1), "+a"(o2), "+a"(o3)
        : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(p), "i"(WAIT));
}

constexpr int kPvBlocks = 2 * kVTiles / 4;  // 8 blocks of 4 MFMAs per 32-key tile

// LDS offsets (relative to va) of block nb's reads: MFMA i = 4 nb + j has
// u = i / 16 (keys 8u..8u+7 of the lane half) and vt = i % 16; MFMAs j = 0, 1
// share column block vt/2 (OFF0), j = 2, 3 the next one (OFF1).
template <int T, int NB>
struct PvOff {
  static constexpr int n0 = 4 * NB, nu = n0 / kVTiles, nvt = n0 % kVTiles;
  static constexpr int row = (32 * T + 8 * nu) * 128;
  static constexpr int off0 = row + 8192 * (nvt >> 1);
  static constexpr int off1 = row + 8192 * ((nvt + 2) >> 1);
};

template <int T, int B>
__device__ __forceinline__ void pv_step(f32x16 (&oacc)[kVTiles], bf16x8 (&ring)[3][4],
                                        const bf16x8 (&pop)[2], const uint32_t (&va)[2][2]) {
  constexpr int u = (4 * B) / kVTiles, vt0 = (4 * B) % kVTiles;
  bf16x8(&cur)[4] = ring[B % 3];
  if constexpr (B + 2 < kPvBlocks) {
    bf16x4 nlo[4], nhi[4];
    pv_block_rd<PvOff<T, B + 2>::off0, PvOff<T, B + 2>::off1, 8>(
        oacc[vt0], oacc[vt0 + 1], oacc[vt0 + 2], oacc[vt0 + 3], nlo, nhi, cur, pop[u], va);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      ring[(B + 2) % 3][j] = __builtin_shufflevector(nlo[j], nhi[j], 0, 1, 2, 3, 4, 5, 6, 7);
  } else if constexpr (B + 1 < kPvBlocks) {
    pv_block_nord<0, false>(oacc[vt0], oacc[vt0 + 1], oacc[vt0 + 2], oacc[vt0 + 3], cur, pop[u]);
  } else {
    pv_block_nord<0, true>(oacc[vt0], oacc[vt0 + 1], oacc[vt0 + 2], oacc[vt0 + 3], cur, pop[u]);
  }
}

template <int T, typename Hook, int... B>
__device__ __forceinline__ void pv_chain(f32x16 (&oacc)[kVTiles], bf16x8 (&ring)[3][4],
                                         const bf16x8 (&pop)[2], const uint32_t (&va)[2][2],
                                         Hook& hook, std::integer_sequence<int, B...>) {
  ((pv_step<T, B>(oacc, ring, pop, va), hook(std::integral_constant<int, B>{})), ...);
}

// Reads of blocks 0 and 1 for tile T; returns with block 0's operands landed
// and block 1's eight reads possibly outstanding.
template <int T>
__device__ __forceinline__ void pv_prologue(bf16x8 (&ring)[3][4], const uint32_t (&va)[2][2]) {
  bf16x4 lo0[4], hi0[4], lo1[4], hi1[4];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%20\n\t"
      "ds_read_b64_tr_b16 %4, %17 offset:%20\n\t"
      "ds_read_b64_tr_b16 %1, %18 offset:%20\n\t"
      "ds_read_b64_tr_b16 %5, %19 offset:%20\n\t"
      "ds_read_b64_tr_b16 %2, %16 offset:%21\n\t"
      "ds_read_b64_tr_b16 %6, %17 offset:%21\n\t"
      "ds_read_b64_tr_b16 %3, %18 offset:%21\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:%21\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:%22\n\t"
      "ds_read_b64_tr_b16 %12, %17 offset:%22\n\t"
      "ds_read_b64_tr_b16 %9, %18 offset:%22\n\t"
      "ds_read_b64_tr_b16 %13, %19 offset:%22\n\t"
      "ds_read_b64_tr_b16 %10, %16 offset:%23\n\t"
      "ds_read_b64_tr_b16 %14, %17 offset:%23\n\t"
      "ds_read_b64_tr_b16 %11, %18 offset:%23\n\t"
      "ds_read_b64_tr_b16 %15, %19 offset:%23\n\t"
      "s_waitcnt lgkmcnt(8)"
      : "=&v"(lo0[0]), "=&v"(lo0[1]), "=&v"(lo0[2]), "=&v"(lo0[3]), "=&v"(hi0[0]), "=&v"(hi0[1]),
        "=&v"(hi0[2]), "=&v"(hi0[3]), "=&v"(lo1[0]), "=&v"(lo1[1]), "=&v"(lo1[2]),
        "=&v"(lo1[3]), "=&v"(hi1[0]), "=&v"(hi1[1]), "=&v"(hi1[2]), "=&v"(hi1[3])
      : "v"(va[0][0]), "v"(va[1][0]), "v"(va[0][1]), "v"(va[1][1]), "i"(PvOff<T, 0>::off0),
        "i"(PvOff<T, 0>::off1), "i"(PvOff<T, 1>::off0), "i"(PvOff<T, 1>::off1));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ring[0][j] = __builtin_shufflevector(lo0[j], hi0[j], 0, 1, 2, 3, 4, 5, 6, 7);
    ring[1][j] = __builtin_shufflevector(lo1[j], hi1[j], 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// O^T += V^T P^T for 32-key tile T: 32 MFMAs in 8 blocks; hook runs after
// each block, as for score_tile.  va[e][par] = page + voff.
template <int T, typename Hook>
__device__ __forceinline__ void pv_tile(f32x16 (&oacc)[kVTiles], const bf16x8 (&pop)[2],
                                        const uint32_t (&va)[2][2], Hook&& hook) {
  bf16x8 ring[3][4];
  pv_prologue<T>(ring, va);
  pv_chain<T>(oacc, ring, pop, va, hook, std::make_integer_sequence<int, kPvBlocks>{});
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

// FP8: the cache holds e4m3 bytes (kv_descale is read); else bf16.
template <bool FP8>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_decode_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
                  const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
                  const int32_t* __restrict__ tile_plan, const int32_t* __restrict__ split_indptr,
                  const float* __restrict__ kv_descale, float* __restrict__ partial_o,
                  float* __restrict__ partial_lse, uint16_t* __restrict__ out,
                  float* __restrict__ lse_out, DecodeParams P) {
  // bf16: two compute buffers.  fp8: compute buffer 0, and two e4m3 staging
  // buffers in the space of compute buffer 1.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kPageBytes];
  constexpr int kSrcPageBytes = FP8 ? kPageBytesF8 : kPageBytes;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int n = lane & 31;      // query row within the wave (B/C column)
  const int h = lane >> 5;      // lane half
  const int part = blockIdx.x;

  const int32_t* tp = tile_plan + part * 8;
  const int b_first = tp[0], pg_first = tp[1], b_last = tp[2], pg_last = tp[3];
  const int first_piece = tp[4], total = tp[5];
  // An empty part, or a row no planner would produce, does nothing (the
  // check is uniform over the work-group, so no wave is left at a barrier).
  if (total <= 0 || b_first < 0 || b_last >= P.bs || b_first > b_last || pg_first < 0 ||
      first_piece < 0)
    return;

  const int row0 = blockIdx.y * kRowsPerBlock + wave * kRowsPerWave;  // first row of this wave
  const int r = row0 + n;                                             // this lane's query row
  const bool wave_active = row0 < P.rows;
  const bool row_valid = r < P.rows;
  const int i_tok = row_valid ? r / P.heads : 0;
  const int i_tok_min = row0 / P.heads;  // smallest token index among the wave's rows

  // ---- per-lane LDS offsets (relative to a page buffer) -------------------
  // Page loads: key i/8 of the group, chunk slot i%8 <- source chunk
  // (i%8) ^ (4 bit4(i) + 2 bit5(i) + bit1(wave)).
  const uint32_t load_voff0 =
      wave * (8 * kRowBytes) + (lane >> 3) * kRowBytes +
      16 * ((lane & 7) ^ (4 * ((lane >> 4) & 1) + 2 * ((lane >> 5) & 1) + ((wave >> 1) & 1)));
  const uint32_t load_voff1 = load_voff0 + 4 * (8 * kRowBytes);  // key group wave + 4
  const uint32_t load_voff_f8 = wave * 1024 + 16 * lane;
  // S^T A operand: lane (m = n, h) reads key 32t + sigma(m) with
  // sigma(8q + 4g + t') = 16g + 4q + t', global chunk 2ks + h, i.e. column
  // block ks/4, chunk 2(ks%4) + h of the block.  Keys 32 apart share the
  // swizzle, so tile 1 is tile 0 plus 32 rows of 128 bytes.
  const int sig = 16 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
  uint32_t koff[4];
  {
    const int sw = 4 * ((sig >> 1) & 1) + 2 * ((sig >> 2) & 1) + ((sig >> 4) & 1);
    const int x = h ^ sw;
#pragma unroll
    for (int i = 0; i < 4; ++i) koff[i] = sig * 128 + (((2 * i) ^ x) << 4);
  }
  // V^T A operand via ds_read_b64_tr_b16: in the 16-lane block (c16, s16)
  // of half h, source lane s16 addresses key kb + 4e + s16/4 (kb a multiple
  // of 8 with bit 4 = h), columns 32vt + 16c16 + 4(s16%4) .. +3; the block
  // then holds column 32vt + 16c16 + s16 of keys kb+4e .. kb+4e+3.
  const int s16 = lane & 15;
  const int c16 = (lane >> 4) & 1;
  uint32_t voff[2][2];  // [e][vt parity]
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int a = s16 >> 2;
    const int sw = 4 * (a >> 1) + 2 * e + h;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int cc = 4 * par + 2 * c16 + ((s16 >> 1) & 1);
      voff[e][par] = (16 * h + 4 * e + a) * 128 + ((cc ^ sw) << 4) + 8 * (s16 & 1);
    }
  }

  // LDS starts as zeros: a load lane that falls outside a page's range may
  // leave its bytes untouched, and those bytes must be finite.
  for (int i = threadIdx.x; i < 2 * kPageBytes / 16; i += kWaves * 64)
    reinterpret_cast<u32x4*>(smem)[i] = (u32x4){0, 0, 0, 0};
  __syncthreads();

  // ---- page cursor for prefetch ----------------------------------------------
  // (nb, np) is the page whose loads are issued next; its block-table entry
  // and length were read one page earlier so the scalar loads never stall.
  int nb = b_first, np = pg_first;
  int nlen = seq_lens[nb];
  int nend = (nb == b_last) ? pg_last : page_count(nlen);
  auto phys_of = [&](int b, int p) -> int64_t {
    if (p >= P.bt_stride) return 0;
    const int64_t pg = block_table[(int64_t)b * P.bt_stride + p];
    return (pg >= 0 && pg < P.num_pages) ? pg : 0;
  };
  int64_t nphys = phys_of(nb, np);
  int nrows = min(kPage, max(0, nlen - np * kPage));
  // Loads of the cursor's page into LDS for page index `j` of the part.
  auto issue = [&](int j) {
    const int vr = __builtin_amdgcn_readfirstlane(nrows);
    if constexpr (FP8)
      issue_loads_f8(std::make_integer_sequence<int, kLoadsPerWaveF8>{},
                     page_rsrc<kD>(kv + nphys * kSrcPageBytes, vr),
                     smem + kPageBytes + (j & 1) * kPageBytesF8, wave, load_voff_f8);
    else
      issue_page_loads(page_rsrc<kRowBytes>(kv + nphys * kSrcPageBytes, vr),
                       smem + (j & 1) * kPageBytes, wave, load_voff0, load_voff1);
  };
  // Move the cursor one page on and read that page's block-table entry and
  // length.  Called after a page's compute, so the scalar loads have a whole
  // barrier interval to land before the next issue needs them.
  auto advance = [&]() {
    ++np;
    while (np >= nend && nb < b_last) {
      ++nb;
      np = 0;
      nlen = seq_lens[nb];
      nend = (nb == b_last) ? pg_last : page_count(nlen);
    }
    nphys = phys_of(nb, np);
    nrows = min(kPage, max(0, nlen - np * kPage));
  };

  issue(0);
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
      if constexpr (FP8) {
        convert_f8_page(smem + kPageBytes + (it & 1) * kPageBytesF8, smem);
        __syncthreads();
      }
    }
    return;
  }

  // Per-tensor dequantisation scale: scores use |delta| in the softmax scale
  // and the sign on q; the output is multiplied by delta.
  const float delta = FP8 ? kv_descale[0] : 1.0f;
  const float c_log2 = P.scale_log2 * fabsf(delta);
  const uint32_t q_sign = (FP8 && delta < 0.f) ? 0x80008000u : 0u;

  bf16x8 qreg[kKSteps];
  f32x16 oacc[kVTiles];
  int it = 0;  // pages of this part processed so far (selects the LDS buffer)
  int cb = b_first;
  int cp = pg_first;
  int piece = first_piece;
  while (true) {
    // ---- one piece: pages [cp, cend) of request cb ---------------------------
    const int32_t L = seq_lens[cb];
    const int cend = (cb == b_last) ? pg_last : page_count(L);
    const int32_t lim = P.causal ? L - P.q_len + i_tok : L - 1;  // last visible key
    // pages from first_masked on may hold keys some row of this wave cannot see
    const int32_t lim_min = P.causal ? L - P.q_len + i_tok_min : L - 1;
    const int first_masked =
        __builtin_amdgcn_readfirstlane(lim_min >= 0 ? (lim_min + 1) / kPage : 0);
    {
      const uint16_t* qrow = q + ((int64_t)cb * P.rows + (row_valid ? r : 0)) * kD + 8 * h;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
        if (FP8) v ^= q_sign;
        if (!row_valid) v = (u32x4){0, 0, 0, 0};
        qreg[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
#pragma unroll
    for (int vt = 0; vt < kVTiles; ++vt) oacc[vt] = (f32x16){};
    float m_run = -INFINITY, l_run = 0.f;

    for (; cp < cend && it < total; ++cp, ++it) {
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads of page `it` landed
      __syncthreads();                     // ... and every wave's; buffer it+1 is free again
      const lds_u8* base = LDS_PTR(uint8_t, smem) + (FP8 ? 0 : (it & 1) * kPageBytes);
      // The next page's loads are issued one per MFMA block (see above):
      // issued back to back they would stall the wave until the address unit
      // drains them.
      const bool has_next = it + 1 < total;
      const __amdgpu_buffer_rsrc_t next_rsrc =
          page_rsrc<FP8 ? kD : kRowBytes>(kv + nphys * kSrcPageBytes,
                                           __builtin_amdgcn_readfirstlane(nrows));
      uint8_t* const next_buf = FP8 ? smem + kPageBytes + ((it + 1) & 1) * kPageBytesF8
                                    : smem + ((it + 1) & 1) * kPageBytes;
      // load K of this wave's share, K < 18 (bf16) or K < 9 (e4m3)
      auto load = [&](auto kc) {
        constexpr int K = decltype(kc)::value;
        if (has_next) {
          if constexpr (FP8)
            issue_one_load_f8<K>(next_rsrc, next_buf, wave, load_voff_f8);
          else
            issue_one_load<K>(next_rsrc, next_buf, wave, load_voff0, load_voff1);
        }
      };
      auto hook_s0 = [&](auto g) { load(g); };
      auto hook_pv0 = [&](auto b) {
        if constexpr (!FP8) load(std::integral_constant<int, 9 + decltype(b)::value>{});
      };
      auto hook_s1 = [&](auto g) {
        if constexpr (!FP8 && decltype(g)::value == 0) load(std::integral_constant<int, 17>{});
      };
      auto no_hook = [](auto) {};
      if constexpr (FP8) {
        convert_f8_page(smem + kPageBytes + (it & 1) * kPageBytesF8, smem);
        __syncthreads();  // the compute page is complete
      }

      // LDS byte addresses of this page's operands
      const uint32_t pbase = (uint32_t)(uintptr_t)base;
      uint32_t ka[4], ka_hi[4], va[2][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ka[i] = pbase + koff[i];
        ka_hi[i] = ka[i] + 32768;
      }
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int par = 0; par < 2; ++par) va[e][par] = pbase + voff[e][par];

#pragma unroll
      for (int t = 0; t < 2; ++t) {
        // ---- S^T = K Q^T for 32-key tile t; sc[i] is key 32t + 16h + i -----------
        f32x16 sc;
        if (t == 0)
          score_tile<0>(sc, ka, ka_hi, qreg, hook_s0);
        else
          score_tile<32 * 128>(sc, ka, ka_hi, qreg, hook_s1);
        // ---- row max of the scaled scores; weights p = 2^(c s - m) -----------------
        // c = softmax_scale * log2(e) > 0, so max(c s) = c max(s).  Keys a row
        // cannot see (causal limit, page tail) are excluded on the pages
        // where they can occur.
        const int key0 = cp * kPage + 32 * t + 16 * h;
        const bool masked = cp >= first_masked;
        float mx[4];
        if (masked) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            mx[j] = -INFINITY;
#pragma unroll
            for (int i = j; i < 16; i += 4)
              mx[j] = fmaxf(mx[j], (key0 + i <= lim) ? sc[i] : -INFINITY);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            mx[j] = fmaxf(fmaxf(sc[j], sc[j + 4]), fmaxf(sc[j + 8], sc[j + 12]));
        }
        const float mloc = xhalf_max(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])));
        const float m_tile = (mloc == -INFINITY) ? -INFINITY : c_log2 * mloc;
        const bool need = m_tile > m_run + kTau;
        if (__any(need)) {
          const float m_new = need ? m_tile : m_run;
          const float alpha = need ? exp2f(m_run - m_new) : 1.0f;
          l_run *= alpha;
          // Rows whose running max is still -inf have o = 0: only a wave with
          // some earlier weight needs the 256-register rescale.
          if (__any(need && m_run != -INFINITY)) {
#pragma unroll
            for (int vt = 0; vt < kVTiles; ++vt) scale_tile(oacc[vt], alpha);
          }
          m_run = m_new;
        }
        const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
        bf16x8 pop[2];
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
        if (masked) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float e = __builtin_amdgcn_exp2f(fmaf(sc[i], c_log2, neg_m));
            const float p = (key0 + i <= lim) ? e : 0.f;
            ls[i & 3] += p;
            pop[i >> 3][i & 7] = (__bf16)p;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sc[i], c_log2, neg_m));
            ls[i & 3] += p;
            pop[i >> 3][i & 7] = (__bf16)p;
          }
        }
        l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
        // ---- O^T += V^T P^T ------------------------------------------------------------
        if (t == 0)
          pv_tile<0>(oacc, pop, va, hook_pv0);
        else
          pv_tile<1>(oacc, pop, va, no_hook);
      }
      if (it + 1 < total) advance();
    }

    // ---- epilogue of the piece ---------------------------------------------------
    {
      const float l_tot = xhalf_sum(l_run);
      const float inv = l_tot > 0.f ? delta / l_tot : 0.f;
      const float lse_val =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
      const int k0 = split_indptr[cb];
      const int k = split_indptr[cb + 1] - k0;
      if (row_valid) {
        const int64_t slot = (int64_t)k0 + piece;
        if (k > 1 && slot < P.partial_slots) {
          float* dst = partial_o + (slot * P.rows + r) * kDv + 4 * h;
#pragma unroll
          for (int vt = 0; vt < kVTiles; ++vt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              float4 v = make_float4(oacc[vt][4 * g] * inv, oacc[vt][4 * g + 1] * inv,
                                     oacc[vt][4 * g + 2] * inv, oacc[vt][4 * g + 3] * inv);
              *reinterpret_cast<float4*>(dst + 32 * vt + 8 * g) = v;
            }
          if (h == 0) partial_lse[slot * P.rows + r] = lse_val;
        } else if (k <= 1) {
          uint16_t* dst = out + ((int64_t)cb * P.rows + r) * kDv + 4 * h;
#pragma unroll
          for (int vt = 0; vt < kVTiles; ++vt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              uint2 v;
              v.x = (uint32_t)f32_to_bf16(oacc[vt][4 * g] * inv) |
                    ((uint32_t)f32_to_bf16(oacc[vt][4 * g + 1] * inv) << 16);
              v.y = (uint32_t)f32_to_bf16(oacc[vt][4 * g + 2] * inv) |
                    ((uint32_t)f32_to_bf16(oacc[vt][4 * g + 3] * inv) << 16);
              *reinterpret_cast<uint2*>(dst + 32 * vt + 8 * g) = v;
            }
          if (lse_out && h == 0) lse_out[(int64_t)cb * P.rows + r] = lse_val;
        }
      }
    }
    if (it >= total || cb >= b_last) break;
    // next request of the part that has pages
    do {
      ++cb;
    } while (cb < b_last && page_count(seq_lens[cb]) <= 0);
    cp = 0;
    piece = 0;
  }
  // Only reached early with a malformed plan: keep the barrier count.
  for (; it < total; ++it) {
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if constexpr (FP8) __syncthreads();
  }
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

extern "C" mla_status mla_decode(const void* q, int32_t bs, int32_t q_len, int32_t num_heads,
                                 const void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                                 const int32_t* block_table, int32_t bt_row_stride,
                                 const int32_t* seq_lens, const int32_t* tile_plan,
                                 int32_t num_parts, const int32_t* split_indptr,
                                 float softmax_scale, int32_t causal, const float* kv_descale,
                                 float* partial_o, float* partial_lse, int32_t partial_slots,
                                 void* out, float* lse, hipStream_t stream) {
  using namespace mla;
  const hipEvent_t ev_start = t_start_event, ev_stop = t_stop_event;
  t_start_event = t_stop_event = nullptr;
  if (!q || !kv_cache || !block_table || !seq_lens || !tile_plan || !split_indptr || !partial_o ||
      !partial_lse || !out)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode: null pointer");
  if (bs <= 0 || q_len <= 0 || num_heads <= 0 || num_pages <= 0 || bt_row_stride <= 0 ||
      num_parts <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode: sizes must be positive");
  if (!finite_nonneg(softmax_scale))
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode: softmax_scale must be finite and >= 0");
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode: unknown kv_dtype");
  if (kv_dtype == MLA_KV_FP8_E4M3 && !kv_descale)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode: fp8 cache needs kv_descale");
  const int64_t rows = (int64_t)q_len * num_heads;
  if (rows < 1 || rows > MLA_MAX_ROWS_PER_REQ)
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode: q_len*num_heads must be in 1..512");
  if (num_parts > MLA_MAX_PARTS)
    return fail(MLA_ERR_CAPACITY, "mla_decode: num_parts above " + std::to_string(MLA_MAX_PARTS));
  if ((int64_t)partial_slots < (int64_t)bs + num_parts)
    return fail(MLA_ERR_CAPACITY, "mla_decode: partial_slots must be at least bs + num_parts");

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
  auto launch = [&](auto kernel, const float* descale) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(q);
    const uint8_t* kvp = reinterpret_cast<const uint8_t*>(kv_cache);
    uint16_t* op = reinterpret_cast<uint16_t*>(out);
    if (ev_start || ev_stop)
      hipExtLaunchKernelGGL(kernel, grid, dim3(kWaves * 64), 0, stream, ev_start, ev_stop, 0, qp,
                            kvp, block_table, seq_lens, tile_plan, split_indptr, descale,
                            partial_o, partial_lse, op, lse, p);
    else
      hipLaunchKernelGGL(kernel, grid, dim3(kWaves * 64), 0, stream, qp, kvp, block_table,
                         seq_lens, tile_plan, split_indptr, descale, partial_o, partial_lse, op,
                         lse, p);
  };
  if (kv_dtype == MLA_KV_FP8_E4M3)
    launch(mla_decode_kernel<true>, kv_descale);
  else
    launch(mla_decode_kernel<false>, nullptr);
  return check_launch("mla_decode");
}
