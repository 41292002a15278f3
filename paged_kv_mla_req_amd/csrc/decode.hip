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
#include <cmath>
#include <utility>

#include "common.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;     // 128
constexpr int kRowBytes = kD * 2;                        // 1152 bytes per bf16 latent row
constexpr int kChunks = kRowBytes / 16;                  // 72 16-byte chunks per row
constexpr int kPageBytes = kPage * kRowBytes;            // 73728
constexpr int kLoadsPerPage = kPageBytes / 1024;         // 72 wave-wide 1 KiB loads
constexpr int kLoadsPerWave = kLoadsPerPage / kWaves;    // 18
constexpr int kKSteps = kD / 16;                         // 36 MFMA k-steps for S
constexpr int kVTiles = kDv / 32;                        // 16 output tiles of 32 columns
constexpr float kTau = 8.0f;                             // lazy-rescale threshold (log2 units)

struct DecodeParams {
  const uint16_t* q;          // bf16 [bs, R, 576]
  const uint8_t* kv;          // [num_pages, 64, 576] bf16
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* tile_plan;
  const int32_t* split_indptr;
  float* partial_o;           // [slots, R, 512]
  float* partial_lse;         // [slots, R]
  uint16_t* out;              // bf16 [bs, R, 512]
  float* lse;                 // [bs, R] or null
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
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t* page, int rows) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(page), (short)0,
                                           rows * kRowBytes, 0x00020000);
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

__device__ __forceinline__ int32_t page_count(int32_t L) {
  return L > 0 ? (L + kPage - 1) / kPage : 0;
}

// S^T chain on MFMA with the accumulator in VGPRs.  The output accumulator
// (16 tiles of 16 fp32) fills all 256 AGPRs, so the score tile must live in
// VGPRs; the compiler selects one accumulator class for every MFMA of a
// kernel, so these MFMAs are issued from inline assembly.  Hazards the
// compiler cannot see are covered by hand: 2 wait states before a group
// (VALU write of an operand -> MFMA read) and 24 after the last MFMA of a
// chain (MFMA write -> VALU read; more than the 18 a 16-pass MFMA needs).
__device__ __forceinline__ void mfma_s4(f32x16& acc, bf16x8 a0, bf16x8 a1, bf16x8 a2, bf16x8 a3,
                                        bf16x8 b0, bf16x8 b1, bf16x8 b2, bf16x8 b3) {
  asm("s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %5, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %6, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %7, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %8, %0"
      : "+v"(acc)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(b0), "v"(b1), "v"(b2), "v"(b3));
}

__device__ __forceinline__ void mfma_s4_last(f32x16& acc, bf16x8 a0, bf16x8 a1, bf16x8 a2,
                                             bf16x8 a3, bf16x8 b0, bf16x8 b1, bf16x8 b2,
                                             bf16x8 b3) {
  asm("s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %5, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %6, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %7, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %8, %0\n\t"
      "s_nop 7\n\t"
      "s_nop 7\n\t"
      "s_nop 7"
      : "+v"(acc)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(b0), "v"(b1), "v"(b2), "v"(b3));
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

__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_decode_bf16_kernel(DecodeParams P) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kPageBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int n = lane & 31;      // query row within the wave (B/C column)
  const int h = lane >> 5;      // lane half
  const int part = blockIdx.x;

  const int32_t* tp = P.tile_plan + part * 8;
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

  // ---- per-lane LDS offsets (relative to a page buffer) -------------------
  // Page loads: key i/8 of the group, chunk slot i%8 <- source chunk
  // (i%8) ^ (4 bit4(i) + 2 bit5(i) + bit1(wave)).
  const uint32_t load_voff0 =
      (wave + 0) * (8 * kRowBytes) + (lane >> 3) * kRowBytes +
      16 * ((lane & 7) ^ (4 * ((lane >> 4) & 1) + 2 * ((lane >> 5) & 1) + ((wave >> 1) & 1)));
  const uint32_t load_voff1 = load_voff0 + 4 * (8 * kRowBytes);  // key group wave + 4
  // S^T A operand: lane (m = n, h) reads key 32t + sigma(m) with
  // sigma(8q + 4g + t') = 16g + 4q + t', global chunk 2ks + h, i.e. column
  // block ks/4, chunk 2(ks%4) + h of the block.
  const int sig = 16 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
  uint32_t koff[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = 32 * t + sig;
    const int sw = 4 * ((key >> 1) & 1) + 2 * ((key >> 2) & 1) + ((key >> 4) & 1);
    const int x = h ^ sw;
#pragma unroll
    for (int i = 0; i < 4; ++i) koff[t][i] = key * 128 + (((2 * i) ^ x) << 4);
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

  // ---- page cursor for prefetch -------------------------------------------
  int nb = b_first, np = pg_first;
  int nlen = P.seq_lens[nb];
  int nend = (nb == b_last) ? pg_last : page_count(nlen);
  auto phys_of = [&](int b, int p) -> int64_t {
    if (p >= P.bt_stride) return 0;
    int64_t pg = P.block_table[(int64_t)b * P.bt_stride + p];
    return (pg >= 0 && pg < P.num_pages) ? pg : 0;
  };
  auto advance = [&]() {
    ++np;
    while (np >= nend && nb < b_last) {
      ++nb;
      np = 0;
      nlen = P.seq_lens[nb];
      nend = (nb == b_last) ? pg_last : page_count(nlen);
    }
  };
  // loads of the page under the prefetch cursor: only its rows below the length
  auto issue_next = [&](uint8_t* buf) {
    const int rows = __builtin_amdgcn_readfirstlane(min(kPage, max(0, nlen - np * kPage)));
    issue_page_loads(page_rsrc(P.kv + phys_of(nb, np) * kPageBytes, rows), buf, wave,
                     load_voff0, load_voff1);
  };

  issue_next(smem);
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
        issue_next(smem + ((it + 1) & 1) * kPageBytes);
        advance();
      }
    }
    return;
  }

  bf16x8 qreg[kKSteps];
  f32x16 oacc[kVTiles];
  int it = 0;  // pages of this part processed so far (selects the LDS buffer)
  int cb = b_first;
  int cp = pg_first;
  int piece = first_piece;
  while (true) {
    // ---- one piece: pages [cp, cend) of request cb ---------------------------
    const int cend = (cb == b_last) ? pg_last : page_count(P.seq_lens[cb]);
    const int32_t L = P.seq_lens[cb];
    const int32_t lim = P.causal ? L - P.q_len + i_tok : L - 1;  // last visible key
    {
      const uint16_t* qrow = P.q + ((int64_t)cb * P.rows + (row_valid ? r : 0)) * kD + 8 * h;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
        if (!row_valid) v = (u32x4){0, 0, 0, 0};
        qreg[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
#pragma unroll
    for (int vt = 0; vt < kVTiles; ++vt) oacc[vt] = (f32x16){};
    float m_run = -INFINITY, l_run = 0.f, lr_run = 0.f;

    for (; cp < cend && it < total; ++cp, ++it) {
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads of page `it` landed
      __syncthreads();                     // ... and every wave's; buffer it+1 is free again
      uint8_t* cur = smem + (it & 1) * kPageBytes;
      if (it + 1 < total) {
        issue_next(smem + ((it + 1) & 1) * kPageBytes);
        advance();
      }

      const uint32_t base = (uint32_t)(uintptr_t)LDS_PTR(uint8_t, cur);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        // ---- S^T = K Q^T for 32-key tile t ---------------------------------------
        f32x16 sc = {};
#pragma unroll
        for (int g = 0; g < kKSteps / 4; ++g) {
          // k-steps 4g .. 4g+3 = column block g, chunks 2i + h
          const uint32_t a = base + 8192 * g;
          bf16x8 k0 = *LDS_PTR(bf16x8, (uintptr_t)(a + koff[t][0]));
          bf16x8 k1 = *LDS_PTR(bf16x8, (uintptr_t)(a + koff[t][1]));
          bf16x8 k2 = *LDS_PTR(bf16x8, (uintptr_t)(a + koff[t][2]));
          bf16x8 k3 = *LDS_PTR(bf16x8, (uintptr_t)(a + koff[t][3]));
          if (g + 1 < kKSteps / 4)
            mfma_s4(sc, k0, k1, k2, k3, qreg[4 * g], qreg[4 * g + 1], qreg[4 * g + 2],
                    qreg[4 * g + 3]);
          else
            mfma_s4_last(sc, k0, k1, k2, k3, qreg[4 * g], qreg[4 * g + 1], qreg[4 * g + 2],
                         qreg[4 * g + 3]);
        }
        // ---- mask, scale, running max ----------------------------------------------
        // sc[i] belongs to key 32t + 16h + i of this page.
        const int key0 = cp * kPage + 32 * t + 16 * h;
        float mloc = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float v = sc[i] * P.scale_log2;
          v = (key0 + i <= lim) ? v : -INFINITY;
          sc[i] = v;
          mloc = fmaxf(mloc, v);
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        const bool need = mloc > m_run + kTau;
        if (__any(need)) {
          const float m_new = need ? mloc : m_run;
          const float alpha = need ? exp2f(m_run - m_new) : 1.0f;
          l_run *= alpha;
          lr_run *= alpha;
#pragma unroll
          for (int vt = 0; vt < kVTiles; ++vt) scale_tile(oacc[vt], alpha);
          m_run = m_new;
        }
        const float mref = (m_run == -INFINITY) ? 0.f : m_run;
        // ---- P = 2^(s - m), row sum, bf16 B operand ---------------------------------
        // Two row sums: of the exact weights (for lse) and of the bf16-rounded
        // weights the MFMA uses (to normalise o, which then stays an exact
        // convex combination of the value rows).
        bf16x8 pop[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2f(sc[i] - mref);
          const __bf16 pb = (__bf16)p;
          l_run += p;
          lr_run += (float)pb;
          pop[i >> 3][i & 7] = pb;
        }
        // ---- O^T += V^T P^T -------------------------------------------------------------
        // MFMA u covers keys 32t + 16h + 8u + 0..7 in lane half h.
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint32_t ub = base + (32 * t + 8 * u) * 128;
#pragma unroll
          for (int vt = 0; vt < kVTiles; ++vt) {
            const uint32_t col = 8192 * (vt >> 1);
            bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                LDS_PTR(bf16x4, (uintptr_t)(ub + voff[0][vt & 1] + col)));
            bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                LDS_PTR(bf16x4, (uintptr_t)(ub + voff[1][vt & 1] + col)));
            bf16x8 vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[vt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[u], oacc[vt], 0, 0, 0);
          }
        }
      }
    }

    // ---- epilogue of the piece ---------------------------------------------------
    {
      const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
      const float lr_tot = lr_run + __shfl_xor(lr_run, 32, 64);
      const float inv = lr_tot > 0.f ? 1.0f / lr_tot : 0.f;
      const float lse_val =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
      const int k0 = P.split_indptr[cb];
      const int k = P.split_indptr[cb + 1] - k0;
      if (row_valid) {
        const int64_t slot = (int64_t)k0 + piece;
        if (k > 1 && slot < P.partial_slots) {
          float* dst = P.partial_o + (slot * P.rows + r) * kDv + 4 * h;
#pragma unroll
          for (int vt = 0; vt < kVTiles; ++vt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              float4 v = make_float4(oacc[vt][4 * g] * inv, oacc[vt][4 * g + 1] * inv,
                                     oacc[vt][4 * g + 2] * inv, oacc[vt][4 * g + 3] * inv);
              *reinterpret_cast<float4*>(dst + 32 * vt + 8 * g) = v;
            }
          if (h == 0) P.partial_lse[slot * P.rows + r] = lse_val;
        } else if (k <= 1) {
          uint16_t* dst = P.out + ((int64_t)cb * P.rows + r) * kDv + 4 * h;
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
          if (P.lse && h == 0) P.lse[(int64_t)cb * P.rows + r] = lse_val;
        }
      }
    }
    if (it >= total || cb >= b_last) break;
    // next request of the part that has pages
    do {
      ++cb;
    } while (cb < b_last && page_count(P.seq_lens[cb]) <= 0);
    cp = 0;
    piece = 0;
  }
  // Only reached early with a malformed plan: keep the barrier count.
  for (; it < total; ++it) {
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  }
}

}  // namespace mla

extern "C" mla_status mla_decode(const void* q, int32_t bs, int32_t q_len, int32_t num_heads,
                                 const void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                                 const int32_t* block_table, int32_t bt_row_stride,
                                 const int32_t* seq_lens, const int32_t* tile_plan,
                                 int32_t num_parts, const int32_t* split_indptr,
                                 float softmax_scale, int32_t causal, const float* kv_descale,
                                 float* partial_o, float* partial_lse, int32_t partial_slots,
                                 void* out, float* lse, hipStream_t stream) {
  using namespace mla;
  if (!q || !kv_cache || !block_table || !seq_lens || !tile_plan || !split_indptr || !partial_o ||
      !partial_lse || !out)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode: null pointer");
  if (bs <= 0 || q_len <= 0 || num_heads <= 0 || num_pages <= 0 || bt_row_stride <= 0 ||
      num_parts <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode: sizes must be positive");
  if (!std::isfinite(softmax_scale))
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode: softmax_scale is not finite");
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
  if (kv_dtype == MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode: fp8 cache not built yet");

  DecodeParams p;
  p.q = reinterpret_cast<const uint16_t*>(q);
  p.kv = reinterpret_cast<const uint8_t*>(kv_cache);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.tile_plan = tile_plan;
  p.split_indptr = split_indptr;
  p.partial_o = partial_o;
  p.partial_lse = partial_lse;
  p.out = reinterpret_cast<uint16_t*>(out);
  p.lse = lse;
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
  hipLaunchKernelGGL(mla_decode_bf16_kernel, grid, dim3(kWaves * 64), 0, stream, p);
  return check_launch("mla_decode");
}
