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

#include "decode_device.h"

namespace mla {

// FP8: the cache holds e4m3 bytes (kv_descale is read); else bf16.  (An
// e4m3 query has a kernel of its own, in decode_q8.hip.)
template <bool FP8>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_decode_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
                  const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
                  const int32_t* __restrict__ tile_plan, const int32_t* __restrict__ split_indptr,
                  const float* __restrict__ kv_descale, uint16_t* __restrict__ partial_o,
                  float* __restrict__ partial_lse, uint16_t* __restrict__ out,
                  float* __restrict__ lse_out, DecodeParams P) {
  // bf16: two compute buffers.  fp8: compute buffer 0, and two e4m3 staging
  // buffers in the space of compute buffer 1.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kPageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stage_all[kWaves][kStageBytes];
  constexpr int kSrcPageBytes = FP8 ? kPageBytesF8 : kPageBytes;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lane = (int)lane_id();  // used before the page loops only
  const int part = part_of_block(blockIdx.x, gridDim.x);

  const int32_t* tp = tile_plan + part * 8;
  const int b_first = tp[0], pg_first = tp[1], b_last = tp[2], pg_last = tp[3];
  const int first_piece = tp[4], total = tp[5];
  // pieces also end at the multiples of tile_cut pages of a request (a packed
  // fixed-tile plan: several tiles of one request in one part are pieces of
  // their own); 0: only where a request ends
  const int tile_cut = tp[6];
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
    if constexpr (FP8)
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
      if constexpr (FP8) {
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
  const float delta = FP8 ? kv_descale[0] : 1.0f;
  // (kept above 0 so that a masked score, -inf, scales to -inf and never to
  // 0 * inf; a zero scale then weights the visible keys equally, to within
  // 1e-30 of a relative error)
  const float c_log2 = fmaxf(P.scale_log2 * fabsf(delta), 1e-30f);
  const uint32_t q_sign = (FP8 && delta < 0.f) ? 0x80008000u : 0u;

  // 36 k-steps of 8 values per lane
  bf16x8 qreg[kKSteps];
  f32x16 oacc[kVTiles];
  // Query rows of request b into qreg.  A lane whose row is past the last one
  // reads row 0 instead: its results stay in that lane's row of the
  // accumulators and are never stored, so no select on the loaded values
  // makes the wave wait for them where they are loaded.
  auto load_q = [&](int b) {
    const uint32_t ql = pinned_lane();
    const int r = row0 + (int)(ql & 31);
    const uint16_t* qrow =
        q + ((int64_t)b * P.rows + (r < P.rows ? r : 0)) * kD + 8 * (int)(ql >> 5);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
      if (FP8) v ^= q_sign;
      qreg[ks] = __builtin_bit_cast(bf16x8, v);
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
  auto park_offsets = [&]() {
    const uint32_t pl = pinned_lane();
    const LaneOffsets o = lane_offsets(pl, wave);
    *reinterpret_cast<u32x4*>(stage_all[wave] + 16 * pl) = (u32x4){o.k, o.v, o.load, pl};
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
    const int req_end = (cb == b_last) ? pg_last : page_count(L);
    const int cend = tile_cut > 0 ? min(req_end, (cp / tile_cut + 1) * tile_cut) : req_end;
    // the next piece is the next tile of this request (same queries)
    const bool same_next = cend < req_end;
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
      if (cp + 1 == cend && it + 1 < total && cb < b_last && !same_next) {
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
      // the page's LDS buffer: the compute page
      const lds_u8* base = LDS_PTR(uint8_t, smem) + (FP8 ? 0 : (it & 1) * kPageBytes);
      // The next page's loads are spread over the MFMA work (issued back to
      // back they would stall the wave until the address unit drains them).
      // Their range (next_rsrc) was worked out on the previous page.  After the
      // part's last page the loads still go out, over an empty range: they
      // only write zeros into the free buffer (and cost no branch per load);
      // the kernel waits for them before it ends.
      uint8_t* const next_buf = FP8 ? smem + kPageBytes + ((it + 1) & 1) * kPageBytesF8
                                    : smem + ((it + 1) & 1) * kPageBytes;
      // load K of this wave's share, K < 18 (bf16) or K < 9 (e4m3)
      auto load = [&](auto kc) {
        constexpr int K = decltype(kc)::value;
        if constexpr (FP8)
          issue_one_load_f8<K>(next_rsrc, next_buf, wave, wave * 1024 + 16 * plane);
        else
          issue_one_load<K>(next_rsrc, next_buf, wave, lo.load, lo.load + 4 * (8 * kRowBytes));
      };
      auto hook_s0 = [&](auto g) { load(g); };
      auto no_hook = [](auto) {};
      if constexpr (FP8) {
        convert_f8_page(smem + kPageBytes + (it & 1) * kPageBytesF8, smem, wave);
        __syncthreads();  // the compute page is complete
      }

      // LDS byte addresses of this page's operands
      const uint32_t pbase = (uint32_t)(uintptr_t)base;
      const uint32_t ka = pbase + lo.k, va = pbase + lo.v;

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
        score_tile<0>(sc0, ka, qreg, hook_s0, NoSlot{});
        // payload slots of the combined chain
        constexpr int kE0 = 5;                 // tile 0, keys 0..7: slots 5..8
        constexpr int kE1 = kCPrefix + 1;      // tile 0, keys 8..15: slots 10, 16, 22, 28
        constexpr int kLd = kCPrefix + 2;      // bf16 loads 9..17: slots 11, 14, .., 35
        constexpr int kM1 = kCLastScore + 1;   // max(1): slots 59..63
        constexpr int kW1 = kM1 + 5;           // tile 1, keys 0..7: slots 64..67
        // (kW1 + 4 == kCSlots: the last branch of pay_c takes every slot from kW1
        // on, so slots past the fourth would weigh keys 8..15 of tile 1 twice)
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
    };

    const int cfast = min(cend, max(cp, first_masked));
    for (; cp < cfast && it < total; ++cp, ++it) page(std::false_type{});
    for (; cp < cend && it < total; ++cp, ++it) page(std::true_type{});

    // ---- epilogue of the piece ---------------------------------------------------
    const bool more = it < total && (cb < b_last || same_next);
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
    if (same_next) {
      ++piece;
    } else {
      cb = ncb;
      cp = 0;
      piece = 0;
    }
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
    uint16_t* op = reinterpret_cast<uint16_t*>(out);
    uint16_t* po = reinterpret_cast<uint16_t*>(partial_o);
    if (ev_start || ev_stop)
      hipExtLaunchKernelGGL(kernel, grid, dim3(kWaves * 64), 0, stream, ev_start, ev_stop, 0, qp,
                            kvp, block_table, seq_lens, tile_plan, split_indptr, kd, po,
                            partial_lse, op, lse, p);
    else
      hipLaunchKernelGGL(kernel, grid, dim3(kWaves * 64), 0, stream, qp, kvp, block_table,
                         seq_lens, tile_plan, split_indptr, kd, po, partial_lse, op, lse, p);
  };
  if (q8)
    launch_decode_q8(grid, stream, ev_start, ev_stop, reinterpret_cast<const uint8_t*>(q),
                     reinterpret_cast<const uint8_t*>(kv_cache), block_table, seq_lens, tile_plan,
                     split_indptr, kv_descale, q_descale, reinterpret_cast<uint16_t*>(partial_o),
                     partial_lse, reinterpret_cast<uint16_t*>(out), lse, p);
  else if (kv_dtype == MLA_KV_FP8_E4M3)
    launch(mla_decode_kernel<true>);
  else
    launch(mla_decode_kernel<false>);
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
