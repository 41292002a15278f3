// MLA decode with an e4m3 query over an e4m3 latent cache (mla_decode_q8).
//
// What it computes: what mla_decode computes (see decode.hip), with the
// query row's value e4m3(code) * q_descale and the cache's latent value
// e4m3(byte) * kv_descale -- the fp8 branch of forward_decode on the FlashMLA
// backend page, which quantises q with scaled_fp8_quant and hands descale_q
// and descale_k to flash_mla_with_kvcache.
//
// How (gfx950), where it differs from the bf16 page kernel:
//  * Both contractions run on v_mfma_f32_32x32x64_f8f6f4 with e4m3 operands,
//    straight from the e4m3 page in LDS: the scores S^T = K Q^T (9 MFMAs per
//    32-key tile) and the output O^T += V^T P^T (one MFMA per 32 value
//    columns and 64 keys).  No page is converted.
//  * The weights p enter the output contraction as two e4m3 numbers, p = hi +
//    lo with hi = e4m3(p) and lo = e4m3(p - hi): two MFMAs into the same
//    accumulator, whose sum carries p to about 2^-8 relative (e4m3 has three
//    mantissa bits; hi leaves at most 2^-4 p, lo rounds that to 2^-4 of
//    itself).  The weights are computed 2^4 larger than exp(s - m) so that the
//    smallest ones stay above e4m3's subnormal range; the row sum carries the
//    same factor, which the normalisation cancels.  The running max moves when
//    a page's max exceeds it by more than 4 (log2), so no weight exceeds
//    2^(4+4) = 256 < 448.
//  * V^T operands come from ds_read_b64_tr_b8: in each 16-lane block a lane
//    receives one column of the 8 keys that the block's lane pairs address, so
//    four reads give a lane the 32 keys of one column in the order of its
//    weights (keys 16h .. 16h+15 and 32+16h .. 32+16h+15 for lane half h, the
//    keys the score layout gives that lane).
//  * Three e4m3 staging buffers (36 KiB each) instead of two bf16 pages: the
//    scores of page i run one page ahead of its output.  Iteration i computes
//    S(i) (the next page's loads spread over its MFMAs), then the output of
//    page i-1 with the softmax of page i (row max, rescale decision, weights,
//    their hi/lo split) in the shadow of those MFMAs.  One barrier per page,
//    before its scores: page i has landed and page i-2's buffer is free for
//    page i+1's loads.
//  * A piece of n pages takes n + 1 iterations (scores only, n - 1 with both
//    chains, output only); its epilogue follows in straight-line code.  The
//    next piece's queries are loaded after the last score MFMA of the piece,
//    as in the bf16 kernel, and the next page's loads are in flight through
//    the output-only iteration and the epilogue.
#include <cmath>
#include <utility>

#include <hip/hip_ext.h>

#include "decode_device.h"

namespace mla {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((__vector_size__(8 * sizeof(uint32_t))));
typedef short s16x2 __attribute__((__vector_size__(2 * sizeof(short))));

constexpr int kKSteps8 = kD / 64;    // 9 score k-steps of 64 columns
constexpr int kK8Ahead = 3;          // score operand reads run 3 MFMAs ahead
constexpr int kK8Ring = kK8Ahead + 1;

constexpr int kStages8 = 3;          // e4m3 staging buffers (page ring)
constexpr float kTau8 = 4.0f;        // largest weight 2^(kTau8 + kPShift) (log2 units)
constexpr float kPShift = 4.0f;      // weights are 2^4 * exp(s - m)
constexpr int kEMax = 64;            // largest output scale exponent of a page
constexpr int kPairs = kVTiles / 2;  // output MFMAs go in pairs of tiles: hi, hi, lo, lo
static_assert(kStages8 * kPageBytesF8 + kWaves * kStageBytes <= 160 * 1024, "LDS budget");

// ---- the e4m3 page in LDS -------------------------------------------------------
// A staging buffer is 9 column blocks of 4 KiB (64 columns of all 64 keys,
// 64 bytes per key); the 16-byte chunk c of key k in a block sits at slot
// c ^ f8_swz(k), f8_swz(k) = bit2(k) + 2 bit4(k), so that the score operand
// reads (32 keys, two chunks each) touch every bank once per 16 lanes.
__device__ __forceinline__ int f8_swz(int k) { return ((k >> 2) & 1) + 2 * ((k >> 4) & 1); }

// Load K of wave w (K < 9) of an e4m3 page into that layout: column block
// K, keys 16w .. 16w + 15; lane i writes slot i % 4 of key 16w + i / 4 from
// global chunk (i % 4) ^ f8_swz(key) (voff, per lane; the column block is the
// immediate offset, which moves the LDS destination too).
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

// LDS offset of lane (m, h)'s score operand (m = lane % 32): key sigma(m)
// (sigma as in lane_offsets: lane (n, h) of the score output then holds keys
// 16 h .. 16 h + 15 of its row), chunk 2h of the column block; chunk 2h + 1
// is at the offset ^ 16.
__device__ __forceinline__ uint32_t k8_offset(uint32_t lane) {
  const int n = lane & 31, h = lane >> 5;
  const int sig = 16 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
  return sig * 64 + (((2 * h) ^ f8_swz(sig)) << 4);
}

// S^T tile (+)= K Q^T over 64 columns, e4m3 operands.
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

template <int... S>
__device__ __forceinline__ void s8_prologue(K8 (&ring)[kK8Ring], uint32_t a0, uint32_t a1,
                                            std::integer_sequence<int, S...>) {
  (k8_read<S>(ring[S], a0, a1), ...);
}

// e4m3 (OCP e4m3fn, round to nearest even) of a and b into bytes 2 HI, 2 HI + 1
// of old, and back.
template <bool HI>
__device__ __forceinline__ uint32_t f8_pack(float a, float b, uint32_t old) {
  return __builtin_bit_cast(
      uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(s16x2, old), a, b,
                                                          1.0f, HI));
}
template <bool HI>
__device__ __forceinline__ f32x2 f8_unpack(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, HI);
}

// O^T tile += V^T P^T over 64 keys, e4m3 operands, accumulator in AGPRs,
// with P^T's column j (query row j) scaled by 2^(sb_j - 127): the scaled
// MFMA takes an E8M0 scale per row of A and per column of B from byte 0 of
// its scale registers (lane j for keys of the first 32-key block, lane j + 32
// for the second), so lane (j, h) holds the scale of row j.  A's scale
// register holds 127 (x 1) in every lane.
__device__ __forceinline__ void mfma_o8(f32x16& o, const u32x8& v, const u32x8& p, uint32_t unit,
                                        uint32_t sb) {
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4"
               : "+a"(o)
               : "v"(v), "v"(p), "v"(unit), "v"(sb));
}

// The V^T operand of tile VT (value columns 32 VT .. 32 VT + 31) of a staged
// page: four transposing reads of 8 keys.  Read j gives lane (column, half h)
// keys 32 (j / 2) + 16 h + 8 (j % 2) .. +7.  vb[par] is the lane's address
// for tiles of parity par (see lane_v8); the column block and j are the
// immediate offset.  Inline assembly, waited for by the chain's own lgkmcnt
// waits: the compiler would put a wait for every page load in flight (vmcnt
// 0) before an LDS read it knows of, since it cannot tell that the loads
// write another buffer.
template <int VT>
__device__ __forceinline__ u32x8 v8_reads(const uint32_t (&vb)[2]) {
  constexpr int OFF = 4096 * (VT >> 1);
  u32x2 r0, r1, r2, r3;
  asm volatile(
      "ds_read_b64_tr_b8 %0, %4 offset:%5\n\t"
      "ds_read_b64_tr_b8 %1, %4 offset:%6\n\t"
      "ds_read_b64_tr_b8 %2, %4 offset:%7\n\t"
      "ds_read_b64_tr_b8 %3, %4 offset:%8"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(vb[VT & 1]), "i"(OFF), "i"(OFF + 512), "i"(OFF + 2048), "i"(OFF + 2560));
  const u32x4 lo = __builtin_shufflevector(r0, r1, 0, 1, 2, 3);
  const u32x4 hi = __builtin_shufflevector(r2, r3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Lane address of the transposing reads, without the page base.  In the
// 16-lane block b = lane / 16 (h = b / 2, column half cb = b % 2) source lane
// t = lane % 16 addresses key 16 h + t / 2 (plus the read's 8-key offset),
// columns 32 VT + 16 cb + 8 (t % 2) .. +7: chunk 2 (VT % 2) + cb of the
// column block VT / 2, at slot chunk ^ f8_swz(key), and the lane's half of
// it.  f8_swz of every key a lane reads is (t / 8) % 2 + 2 h.
__device__ __forceinline__ uint32_t lane_v8(uint32_t lane, int par) {
  const int t = lane & 15, cb = (lane >> 4) & 1, h = lane >> 5;
  const int key = 16 * h + (t >> 1);
  const int swz = ((t >> 3) & 1) + 2 * h;
  return key * 64 + (((2 * par + cb) ^ swz) << 4) + 8 * (t & 1);
}

// ---- the score chain: S^T of both key tiles of a page, 18 MFMAs -------------
// Step S = MFMA S, pay(S), the operand read of step S + kK8Ahead, the wait
// for S + 1, hook(S).
template <int S, typename Hook, typename Pay>
__device__ __forceinline__ void sx_step(f32x16& sc0, f32x16& sc1, K8 (&ring)[kK8Ring],
                                        const u32x8 (&qreg)[kKSteps8], uint32_t a0, uint32_t a1,
                                        Hook& hook, Pay& pay) {
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
__device__ __forceinline__ void sx_steps(f32x16& sc0, f32x16& sc1, K8 (&ring)[kK8Ring],
                                         const u32x8 (&qreg)[kKSteps8], uint32_t a0, uint32_t a1,
                                         Hook& hook, Pay& pay, std::integer_sequence<int, S...>) {
  (sx_step<S>(sc0, sc1, ring, qreg, a0, a1, hook, pay), ...);
}

template <typename Hook, typename Pay>
__device__ __forceinline__ void score_chain8(f32x16& sc0, f32x16& sc1,
                                             const u32x8 (&qreg)[kKSteps8], uint32_t ka,
                                             Hook&& hook, Pay&& pay) {
  const uint32_t a1 = ka ^ 16u;
  K8 ring[kK8Ring];
  s8_prologue(ring, ka, a1, std::make_integer_sequence<int, kK8Ahead>{});
  lgkm_wait<2 * (kK8Ahead - 1)>();
  MLA_SB();
  sx_steps(sc0, sc1, ring, qreg, ka, a1, hook, pay,
           std::make_integer_sequence<int, 2 * kKSteps8>{});
}

// ---- the output chain: O^T += V^T P^T over one page, 32 MFMAs ---------------
// Pair U (tiles 2U and 2U + 1): the V^T reads of pair U + 1, the wait for
// pair U's, then MFMAs hi(2U), hi(2U+1), lo(2U), lo(2U+1) with payload slots
// 4U .. 4U + 3 after them (lo(t) accumulates onto hi(t) one MFMA later).
template <int U, typename Pay>
__device__ __forceinline__ void o8_pair(f32x16 (&oacc)[kVTiles], u32x8 (&ring)[2][2],
                                        const u32x8& phi, const u32x8& plo, uint32_t unit,
                                        uint32_t sb, const uint32_t (&vb)[2], Pay& pay) {
  if constexpr (U + 1 < kPairs) {
    ring[(U + 1) % 2][0] = v8_reads<2 * U + 2>(vb);
    ring[(U + 1) % 2][1] = v8_reads<2 * U + 3>(vb);
    MLA_SB();
    lgkm_wait<8>();  // pair U's eight reads landed (pair U + 1's still in flight)
  } else {
    lgkm_wait<0>();
  }
  MLA_SB();
  const u32x8 va = ring[U % 2][0], vb2 = ring[U % 2][1];
  mfma_o8(oacc[2 * U], va, phi, unit, sb);
  MLA_SB();
  pay(ic<4 * U>{});
  MLA_SB();
  mfma_o8(oacc[2 * U + 1], vb2, phi, unit, sb);
  MLA_SB();
  pay(ic<4 * U + 1>{});
  MLA_SB();
  mfma_o8(oacc[2 * U], va, plo, unit, sb);
  MLA_SB();
  pay(ic<4 * U + 2>{});
  MLA_SB();
  mfma_o8(oacc[2 * U + 1], vb2, plo, unit, sb);
  MLA_SB();
  pay(ic<4 * U + 3>{});
  MLA_SB();
}

template <typename Pay, int... U>
__device__ __forceinline__ void o8_pairs(f32x16 (&oacc)[kVTiles], u32x8 (&ring)[2][2],
                                         const u32x8& phi, const u32x8& plo, uint32_t unit,
                                         uint32_t sb, const uint32_t (&vb)[2], Pay& pay,
                                         std::integer_sequence<int, U...>) {
  (o8_pair<U>(oacc, ring, phi, plo, unit, sb, vb, pay), ...);
}

// vb: the page's lane addresses for even and odd tiles (LDS byte addresses);
// unit, sb: the scale registers of mfma_o8.
template <typename Pay>
__device__ __forceinline__ void output_chain8(f32x16 (&oacc)[kVTiles], const u32x8& phi,
                                              const u32x8& plo, uint32_t unit, uint32_t sb,
                                              const uint32_t (&vb)[2], Pay&& pay) {
  u32x8 ring[2][2];
  ring[0][0] = v8_reads<0>(vb);
  ring[0][1] = v8_reads<1>(vb);
  MLA_SB();
  o8_pairs(oacc, ring, phi, plo, unit, sb, vb, pay, std::make_integer_sequence<int, kPairs>{});
  mfma_tail();
  MLA_SB();
}

// f(ic<K>) for K in order.
template <typename F, int... K>
__device__ __forceinline__ void each_slot(F& f, std::integer_sequence<int, K...>) {
  (f(ic<K>{}), ...);
}


// This wave's 32 rows of o * scale to dst as bf16 rows of 512 values (row r
// at dst + r * 512), rows at or past `rows` left out.  Each tile (32 columns)
// goes to the wave's LDS area straight from the accumulator registers (the
// 16-byte chunk c of row n at c ^ (n % 8)) and leaves row-major: lane i reads
// 4 values of row 8 qq + i / 8, scales, converts and stores them, so that a
// store covers 8 rows x 64 bytes.  One tile is in flight at a time, to keep
// the registers this takes small (the next piece's queries stay live).
__device__ __forceinline__ void store_rows8(const f32x16 (&oacc)[kVTiles], float scale,
                                            uint8_t* stage, uint16_t* dst, int row0, int rows,
                                            uint32_t lane) {
  const int n = lane & 31, h = lane >> 5, j = lane & 7;
  const uint32_t sbase = (uint32_t)(uintptr_t)LDS_PTR(uint8_t, stage);
  uint32_t wa[4], ra[4], go[4];
  float rs[4];
  bool ok[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) wa[g] = sbase + n * 128 + (((2 * g + h) ^ (n & 7)) << 4);
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int row = 8 * qq + (int)(lane >> 3);
    rs[qq] = __shfl(scale, row);
    ra[qq] = sbase + row * 128 + ((j ^ (row & 7)) << 4);
    go[qq] = (uint32_t)((row0 + row) * kDv + 4 * j);
    ok[qq] = row0 + row < rows;
  }
#pragma unroll
  for (int p = 0; p < kVTiles; ++p) {
    const f32x16& t = oacc[p];
    *LDS_PTR(f32x4, (uintptr_t)wa[0]) = __builtin_shufflevector(t, t, 0, 1, 2, 3);
    *LDS_PTR(f32x4, (uintptr_t)wa[1]) = __builtin_shufflevector(t, t, 4, 5, 6, 7);
    *LDS_PTR(f32x4, (uintptr_t)wa[2]) = __builtin_shufflevector(t, t, 8, 9, 10, 11);
    *LDS_PTR(f32x4, (uintptr_t)wa[3]) = __builtin_shufflevector(t, t, 12, 13, 14, 15);
    // (read as float vectors: clang's __builtin_bit_cast of a subscripted
    // vector element reads element 0)
    f32x4 v[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) v[qq] = *LDS_PTR(f32x4, (uintptr_t)ra[qq]);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const float x0 = v[qq][0] * rs[qq], x1 = v[qq][1] * rs[qq];
      const float x2 = v[qq][2] * rs[qq], x3 = v[qq][3] * rs[qq];
      const uint32_t lo =
          __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x0, x1}, bf16x2));
      const uint32_t hi =
          __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x2, x3}, bf16x2));
      if (ok[qq]) *reinterpret_cast<uint2*>(dst + go[qq] + 32 * p) = make_uint2(lo, hi);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace

// One part of the plan per work-group (grid.x) and 128 query rows (grid.y),
// as the bf16 page kernel; q holds e4m3 codes.
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_decode_q8_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ kv,
                     const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
                     const int32_t* __restrict__ tile_plan,
                     const int32_t* __restrict__ split_indptr,
                     const float* __restrict__ kv_descale, const float* __restrict__ q_descale,
                     uint16_t* __restrict__ partial_o, float* __restrict__ partial_lse,
                     uint16_t* __restrict__ out, float* __restrict__ lse_out, DecodeParams P) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage8[kStages8][kPageBytesF8];
  __shared__ __attribute__((aligned(16))) uint8_t stage_all[kWaves][kStageBytes];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = (int)lane_id();
  const int part = part_of_block(blockIdx.x, gridDim.x);
  const int32_t* tp = tile_plan + part * 8;
  const int b_first = tp[0], pg_first = tp[1], b_last = tp[2], pg_last = tp[3];
  const int first_piece = tp[4], total = tp[5];
  // pieces also end at the multiples of tile_cut pages of a request (packed
  // fixed-tile plan); 0: only where a request ends
  const int tile_cut = tp[6];
  if (total <= 0 || b_first < 0 || b_last >= P.bs || b_first > b_last || pg_first < 0 ||
      first_piece < 0)
    return;

  const int row0 = blockIdx.y * kRowsPerBlock + wave * kRowsPerWave;
  const bool wave_active = row0 < P.rows;
  const int i_tok_min = row0 / P.heads;

  // LDS starts as zeros (a load lane outside a page's range may leave its
  // bytes untouched; they must be finite).
  for (int i = wave * 64 + lane; i < kStages8 * kPageBytesF8 / 16; i += kWaves * 64)
    reinterpret_cast<u32x4*>(&stage8[0][0])[i] = (u32x4){0, 0, 0, 0};
  __syncthreads();

  // ---- page cursor for the loads (as in the bf16 kernel) ----------------------
  int nb = b_first, np = pg_first;
  int nlen = uniform_load(seq_lens, nb);
  int nend = (nb == b_last) ? pg_last : page_count(nlen);
  auto raw_of = [&](int b, int p) -> int32_t {
    return p < P.bt_stride ? block_table[(int64_t)b * P.bt_stride + p] : -1;
  };
  int32_t nraw = raw_of(nb, np);
  auto cursor_bad = [&]() -> uint32_t { return (nraw >= 0 && nraw < P.num_pages) ? 0u : 1u; };
  auto nphys = [&]() -> int64_t { return cursor_bad() ? 0 : nraw; };
  int nrows = min(kPage, max(0, nlen - np * kPage));
  auto stage_of = [&](int j) -> uint8_t* { return &stage8[j % kStages8][0]; };
  auto issue = [&](int j) {
    const int vr = __builtin_amdgcn_readfirstlane(cursor_bad() ? 0 : nrows);
    issue_loads_q8(std::make_integer_sequence<int, kKSteps8>{},
                   page_rsrc<kD>(kv + nphys() * kPageBytesF8, vr), stage_of(j), wave,
                   q8_load_offset(lane, wave));
  };
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
  uint32_t badq = cursor_bad();  // bit 0: page it is a bad one; bit 1: page it + 1
  advance();

  // Every wave passes exactly total barriers (one per page, before its
  // scores).
  if (!wave_active) {
    for (int it = 0; it < total; ++it) {
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
      if (it + 1 < total) {
        issue(it + 1);
        advance();
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);
    return;
  }

  __amdgpu_buffer_rsrc_t next_rsrc;
  auto next_range = [&](bool has) -> uint32_t {
    const uint32_t bad = has ? cursor_bad() : 0u;
    next_rsrc = page_rsrc<kD>(kv + nphys() * kPageBytesF8,
                              (has && !bad) ? __builtin_amdgcn_readfirstlane(nrows) : 0);
    return bad;
  };
  badq |= next_range(1 < total) << 1;
  if (1 < total) advance();

  // scales: |q_descale * kv_descale| in the base-2 softmax scale and its sign
  // on the query codes; kv_descale on the output
  const float delta = kv_descale[0];
  const float qk = delta * q_descale[0];
  const float c_log2 = fmaxf(P.scale_log2 * fabsf(qk), 1e-30f);
  const uint32_t q_sign = qk < 0.f ? 0x80808080u : 0u;

  u32x8 qreg[kKSteps8];
  f32x16 oacc[kVTiles];
  auto load_q = [&](int b) {
    const uint32_t ql = pinned_lane();
    const int r = row0 + (int)(ql & 31);
    const uint8_t* qrow =
        q + ((int64_t)b * P.rows + (r < P.rows ? r : 0)) * kD + 32 * (int)(ql >> 5);
#pragma unroll
    for (int ks = 0; ks < kKSteps8; ++ks) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(qrow + 64 * ks) ^ q_sign;
      const u32x4 hi = *reinterpret_cast<const u32x4*>(qrow + 64 * ks + 16) ^ q_sign;
      qreg[ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };

  // score side: the page `it` (request cb, page cp of it, piece `piece`)
  int cb = b_first, cp = pg_first, piece = first_piece;
  int32_t L = uniform_load(seq_lens, cb);
  int req_end = (cb == b_last) ? pg_last : page_count(L);
  auto tile_end = [&](int page) {
    return tile_cut > 0 ? min(req_end, (page / tile_cut + 1) * tile_cut) : req_end;
  };
  int cend = tile_end(cp);
  auto first_masked_of = [&](int32_t len) {
    const int32_t lim_min = P.causal ? len - P.q_len + i_tok_min : len - 1;
    return __builtin_amdgcn_readfirstlane(lim_min >= 0 ? (lim_min + 1) / kPage : 0);
  };
  int first_masked = first_masked_of(L);
  // m_ref: the row's reference max of the piece (log2 units); l_run: the sum
  // of its weights, each page's scaled by 2^e of that page
  float m_ref = -INFINITY, l_run = 0.f;
  // output side: the piece of page it - 1, when that page ended it
  bool pv_last = false;
  int pv_cb = cb, pv_piece = piece;
  float pv_m = -INFINITY, pv_l = 0.f;
  bool first_wait = true;

  load_q(cb);
  zero_acc(oacc);
  __builtin_amdgcn_s_waitcnt(0x0f70);

  // weights of the page being scored: hi/lo for the output chain of the next
  // iteration (cur: the ones the output chain of this iteration uses)
  u32x8 phi_cur = {}, plo_cur = {}, phi_nxt = {}, plo_nxt = {};
  // their output scale (E8M0 127 + e in byte 0) and e
  uint32_t sb_cur = 127u, sb_nxt = 127u;
  int e_nxt = 0;
  uint32_t unit = 0x7f7f7f7fu;
  asm volatile("" : "+v"(unit));
  f32x16 sc0, sc1;
  float alpha = 1.f;
  bool need = false;

  // One iteration: the scores of page it (has_s) and the output of page
  // it - 1 (has_o).  A piece of n pages takes n + 1 iterations: scores only,
  // n - 1 with both chains, output only; the epilogue follows the last one in
  // straight-line code.  Each kind is an instance of its own, so that no
  // chain sits in a branch (a branch around a chain, or an epilogue inside
  // the steady-state loop, makes the register allocator move the output
  // accumulators between register files).
  int it = 0;
  auto iterate = [&](auto has_s_c, auto has_o_c) {
    constexpr bool has_s = decltype(has_s_c)::value;
    constexpr bool has_o = decltype(has_o_c)::value;
    if constexpr (has_s) {
      // page it has landed; the buffer of page it + 1 held page it - 2, whose
      // output ran before this barrier
      if (first_wait) __builtin_amdgcn_s_waitcnt(0x0f70);
      first_wait = true;
      __syncthreads();
    }
    const bool bad = badq & 1u;
    const uint32_t pl = pinned_lane();
    const uint32_t s_base = (uint32_t)(uintptr_t)LDS_PTR(uint8_t, stage_of(it));
    const uint32_t o_base = (uint32_t)(uintptr_t)LDS_PTR(uint8_t, stage_of(it + kStages8 - 1));
    uint8_t* const next_buf = stage_of(it + 1);

    // ---- scores of page it, the next page's loads in the shadow ---------------
    if constexpr (has_s) {
      const uint32_t ka = s_base + k8_offset(pl);
      const uint32_t voff = q8_load_offset(pl, wave);
      auto hook = [&](auto step) {
        constexpr int k = decltype(step)::value;
        if constexpr (k < kKSteps8) issue_one_load_q8<k>(next_rsrc, next_buf, wave, voff);
      };
      score_chain8(sc0, sc1, qreg, ka, hook, NoSlot{});
      // the piece's last page: its queries are no longer needed; load the next
      // piece's (waited for here, with the next page's loads)
      if (cp + 1 == cend && it + 1 < total && cb < b_last && cend == req_end) {
        int ncb = cb;
        do {
          ++ncb;
        } while (ncb < b_last && page_count(uniform_load(seq_lens, ncb)) <= 0);
        load_q(ncb);
        __builtin_amdgcn_s_waitcnt(0x0f70);
      }
    }

    // ---- softmax of page it, in slots --------------------------------------------
    // sc0[i] / sc1[i] is key 16h + i of key tile 0 / 1 of the lane's row.
    const bool masked = has_s && (cp >= first_masked || bad);
    int vis0 = 16, vis1 = 16;
    if (masked) {
      const int r = row0 + (int)(pl & 31);
      const int i_tok = r < P.rows ? r / P.heads : 0;
      const int32_t lim = P.causal ? L - P.q_len + i_tok : L - 1;
      vis0 = bad ? 0 : lim - (cp * kPage + 16 * (int)(pl >> 5)) + 1;
      vis1 = vis0 - 32;
    }
    float mx[4], ls[4];
    float m_tile = 0.f, neg_m = 0.f;
    float p[32];
    auto softmax_slot = [&](auto slot) {
      constexpr int k = decltype(slot)::value;
      if constexpr (k == 0) {
        if (masked) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sc0[i] = i < vis0 ? sc0[i] : -INFINITY;
        }
      } else if constexpr (k == 1) {
        if (masked) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sc1[i] = i < vis1 ? sc1[i] : -INFINITY;
        }
      } else if constexpr (k >= 2 && k < 6) {
        // row max, in four parts of eight values
        constexpr int g = k - 2;
        const f32x16& sc = g < 2 ? sc0 : sc1;
        constexpr int o = 8 * (g & 1);
        mx[g] = fmaxf(fmaxf(fmaxf(sc[o], sc[o + 1]), fmaxf(sc[o + 2], sc[o + 3])),
                      fmaxf(fmaxf(sc[o + 4], sc[o + 5]), fmaxf(sc[o + 6], sc[o + 7])));
        keep(mx[g]);
      } else if constexpr (k == 6) {
        m_tile = c_log2 * xhalf_max(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])));
        keep(m_tile);
      } else if constexpr (k == 7) {
        // the page's weights are 2^(s - m_ref - e + kPShift), e >= 0 the
        // least integer that keeps them <= 2^(kTau8 + kPShift), and its
        // output MFMAs scale them back by 2^e: O stays relative to the
        // piece's m_ref (its first finite page max) and is not rescaled,
        // unless e would exceed kEMax; then m_ref moves to the page's max -
        // kTau8 and O follows after this chain
        if (m_ref == -INFINITY) m_ref = m_tile;
        const float over = m_ref == -INFINITY ? -1.f : m_tile - m_ref - kTau8;
        int e = over > 0.f ? (int)__builtin_ceilf(over) : 0;
        need = e > kEMax;
        const float m_new = need ? m_tile - kTau8 : m_ref;
        alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
        l_run *= alpha;
        m_ref = m_new;
        e = need ? 0 : e;
        e_nxt = e;
        sb_nxt = 127u + (uint32_t)e;
        neg_m = (m_ref == -INFINITY ? 0.f : -(m_ref + (float)e)) + kPShift;
#pragma unroll
        for (int j = 0; j < 4; ++j) ls[j] = 0.f;
      } else if constexpr (k >= 8 && k < 32) {
        // weights of dword d (values 4d .. 4d + 3) in three slots: values,
        // their hi codes and values, the lo codes
        constexpr int d = (k - 8) / 3, part = (k - 8) % 3;
        if constexpr (part == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * d + e;
            const float s = i < 16 ? sc0[i] : sc1[i - 16];
            p[i] = __builtin_amdgcn_exp2f(fmaf(s, c_log2, neg_m));
            ls[e] += p[i];
          }
          keep(p[4 * d]), keep(p[4 * d + 1]), keep(p[4 * d + 2]), keep(p[4 * d + 3]);
        } else if constexpr (part == 1) {
          uint32_t w = f8_pack<false>(p[4 * d], p[4 * d + 1], 0u);
          w = f8_pack<true>(p[4 * d + 2], p[4 * d + 3], w);
          phi_nxt[d] = w;
          keep(w);
        } else {
          const f32x2 h0 = f8_unpack<false>(phi_nxt[d]), h1 = f8_unpack<true>(phi_nxt[d]);
          uint32_t w = f8_pack<false>(p[4 * d] - h0.x, p[4 * d + 1] - h0.y, 0u);
          w = f8_pack<true>(p[4 * d + 2] - h1.x, p[4 * d + 3] - h1.y, w);
          plo_nxt[d] = w;
          keep(w);
        }
      }
    };

    // ---- output of page it - 1, the softmax of page it in its slots ----------
    if constexpr (has_o) {
      const uint32_t vb[2] = {o_base + lane_v8(pl, 0), o_base + lane_v8(pl, 1)};
      auto pay = [&](auto slot) {
        constexpr int k = decltype(slot)::value;
        if constexpr (has_s) {
          softmax_slot(slot);
          if constexpr (k == 17) {
            // the range of page it + 2, loaded during iteration it + 1
            badq = (badq >> 1) | (next_range(it + 2 < total) << 1);
          } else if constexpr (k == 21) {
            if (it + 2 < total) advance();
          }
        }
      };
      output_chain8(oacc, phi_cur, plo_cur, unit, sb_cur, vb, pay);
    } else {
      each_slot(softmax_slot, std::make_integer_sequence<int, 32>{});
      badq = (badq >> 1) | (next_range(it + 2 < total) << 1);
      if (it + 2 < total) advance();
    }
    if constexpr (has_s) l_run += __builtin_ldexpf((ls[0] + ls[1]) + (ls[2] + ls[3]), e_nxt);

    // ---- after the output chain: the rescale of O --------------------------------
    if (has_o && has_s && __any(need)) {  // (compile-time has_o, has_s)
      // the reference max moved for page it: O (through page it - 1) follows
#pragma unroll
      for (int vt = 0; vt < kVTiles; ++vt) scale_tile(oacc[vt], alpha);
    }

    // ---- move the score side on ---------------------------------------------------
    pv_last = false;
    if (has_s) {
      if (cp + 1 == cend || it + 1 == total) {
        // page it ends its piece: its output (next iteration) ends it
        pv_last = true;
        pv_cb = cb;
        pv_piece = piece;
        pv_m = m_ref;
        pv_l = l_run;
        m_ref = -INFINITY;
        l_run = 0.f;
        if (cend < req_end) {
          // the next tile of the same request (same queries)
          ++cp;
          ++piece;
          cend = tile_end(cp);
        } else {
          if (cb < b_last) {
            do {
              ++cb;
              L = uniform_load(seq_lens, cb);
            } while (cb < b_last && page_count(L) <= 0);
            req_end = (cb == b_last) ? pg_last : page_count(L);
            first_masked = first_masked_of(L);
          }
          cp = 0;
          piece = 0;
          cend = tile_end(cp);
        }
      } else {
        ++cp;
      }
    }
    phi_cur = phi_nxt;
    plo_cur = plo_nxt;
    sb_cur = sb_nxt;
  };
  using T = std::true_type;
  using F = std::false_type;
  while (it < total) {
    iterate(T{}, F{});
    ++it;
    while (!pv_last) {
      iterate(T{}, T{});
      ++it;
    }
    iterate(F{}, T{});
    // the piece's outputs
    const uint32_t pl = pinned_lane();
    const bool more = it < total;
    if (more) {
      // the next page's loads land before any store goes out
      __builtin_amdgcn_s_waitcnt(0x0f70);
      first_wait = false;
    }
    const float l_tot = xhalf_sum(pv_l);
    const float inv = l_tot > 0.f ? delta / l_tot : 0.f;
    const float lse_val =
        l_tot > 0.f ? (pv_m + log2f(l_tot) - kPShift) * 0.69314718055994531f : -INFINITY;
    const int k0 = uniform_load(split_indptr, pv_cb);
    const int kk = uniform_load(split_indptr, pv_cb + 1) - k0;
    const int64_t slot = (int64_t)k0 + pv_piece;
    const bool to_partial = kk > 1;
    const int r = row0 + (int)(pl & 31);
    // a slot outside the partial buffer stores nothing (rows = 0)
    const bool st = !to_partial || (slot >= 0 && slot < P.partial_slots);
    float* const lp = to_partial ? partial_lse + slot * P.rows
                                 : (lse_out ? lse_out + (int64_t)pv_cb * P.rows : nullptr);
    if (st && lp && (pl >> 5) == 0 && r < P.rows) lp[r] = lse_val;
    uint16_t* const ob = to_partial ? partial_o + slot * P.rows * kDv
                                    : out + (int64_t)pv_cb * P.rows * kDv;
    store_rows8(oacc, inv, stage_all[wave], ob, row0, st ? P.rows : 0, pl);
    if (more) zero_acc(oacc);
  }
  // the last loads land before the work-group's LDS is released
  __builtin_amdgcn_s_waitcnt(0x0f70);
}

void launch_decode_q8(dim3 grid, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop,
                      const uint8_t* q, const uint8_t* kv, const int32_t* block_table,
                      const int32_t* seq_lens, const int32_t* tile_plan,
                      const int32_t* split_indptr, const float* kv_descale,
                      const float* q_descale, uint16_t* partial_o, float* partial_lse,
                      uint16_t* out, float* lse, const DecodeParams& p) {
  if (ev_start || ev_stop)
    hipExtLaunchKernelGGL(mla_decode_q8_kernel, grid, dim3(kWaves * 64), 0, stream, ev_start,
                          ev_stop, 0, q, kv, block_table, seq_lens, tile_plan, split_indptr,
                          kv_descale, q_descale, partial_o, partial_lse, out, lse, p);
  else
    hipLaunchKernelGGL(mla_decode_q8_kernel, grid, dim3(kWaves * 64), 0, stream, q, kv,
                       block_table, seq_lens, tile_plan, split_indptr, kv_descale, q_descale,
                       partial_o, partial_lse, out, lse, p);
}

}  // namespace mla
