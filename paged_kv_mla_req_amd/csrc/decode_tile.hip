// MLA decode over a paged latent cache, split along the KV sequence (gfx950).
//
// What it computes: for each request b and query row r (token i, head h),
// softmax attention of the 576-wide absorbed query over the request's latent
// rows 0..L_b-1 (bottom-right causal for q_len > 1), with V the first 512
// columns of the same latent row: what the FlashMLA backend page's
// forward_decode (and the target-verify branch of forward_extend) asks of
// flash_mla_with_kvcache -- k_cache viewed as [-1, 64, 1, 576],
// head_dim_v = kv_lora_rank, softmax_scale = layer.scaling, causal = True.
//
// How:
//  * A work-group of 4 waves (one per SIMD) takes one planner part (grid.x)
//    and a block of 128 query rows (grid.y).  It walks the part's keys in
//    tiles of 32 (half a page); every tile is staged once in LDS and shared
//    by all 128 rows (all heads of a request read one latent row per token).
//  * The scores are split by rows, the output by columns.  Wave w computes
//    S^T = K Q^T for rows 32w .. 32w+31 (its queries live in 144 VGPRs),
//    their masked online softmax, and writes the weights P to LDS; it then
//    adds V^T P^T for value columns 128w .. 128w+127 of all 128 rows (16
//    accumulator tiles of 32 x 32, 256 AGPRs), reading the four row groups'
//    weights from LDS.  A value operand (32 columns x 16 keys, two
//    transposing LDS reads) then feeds four MFMAs, so each wave reads a
//    quarter of the value columns instead of all of them: the LDS reads that
//    bounded the row-only split are cut by about a third.
//  * The output MFMAs of a tile run in the next tile's interval, in one
//    straight-line chain with the next tile's score MFMAs (68 MFMAs per
//    interval: 36 score, 32 output); the softmax runs in the shadow of the
//    last 16 output MFMAs.  One work-group barrier per tile publishes the
//    tile's data, the weights and the rescale factors.
//  * Tiles move HBM -> LDS by direct-to-LDS 16-byte buffer loads (9 per wave
//    per tile, spread through the chain), two tiles ahead: a ring of four
//    32 KiB slots holds the value columns (tile t-1 for the output MFMAs, t
//    for the scores, t+1 and t+2 landing) and a ring of three 4 KiB slots the
//    rope columns 512..575 (scores only).  The load range stops at the
//    request's last key: key slots past it arrive as zeros (or keep earlier
//    finite tile data) and their scores are masked.
//
// The LDS layout of a tile: 9 column blocks of 4 KiB (64 columns of the 32
// keys, 128 bytes per key); the 16-byte chunk c of key k sits at chunk
// c ^ swz(k), swz(k) = 4 bit1(k) + 2 bit2(k) + bit4(k).  With it the 16-byte
// key reads of the score MFMA and the transposing value reads of the output
// MFMA (ds_read_b64_tr_b16) hit each bank once per access group.
#include <cmath>
#include <utility>

#include <hip/hip_ext.h>

#include "common.h"
#include "decode_tile.h"

namespace mla {
namespace tile {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define LDS_AT(T, a) ((__attribute__((address_space(3))) T*)(uintptr_t)(a))
#define SB() __builtin_amdgcn_sched_barrier(0)

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;                 // 256
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;  // 128
constexpr int kGroups = kWaves;                       // row groups of 32
constexpr int kCTiles = 4;                            // a wave's 32-column output tiles
constexpr int kTileKeys = 32;
constexpr int kRowBytes = kD * 2;                     // 1152
constexpr int kBlockBytes = kTileKeys * 128;          // 4096: 64 columns of a tile
constexpr int kVSlotBytes = 8 * kBlockBytes;          // 32768: value columns of a tile
constexpr int kVSlots = 4;
constexpr int kRopeSlots = 3;
constexpr int kRopeBase = kVSlots * kVSlotBytes;                 // 131072
constexpr int kPBase = kRopeBase + kRopeSlots * kBlockBytes;     // 143360
constexpr int kPBufBytes = kGroups * 2 * 1024;                   // weights of one tile: 8 KiB
constexpr int kABase = kPBase + 2 * kPBufBytes;                  // rescale factors [n][g]
constexpr int kIBase = kABase + 2 * 512;                         // output scales [n][g]
constexpr int kLdsBytes = kIBase + 2 * 512;                      // 161792
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
constexpr int kKSteps = kD / 16;       // 36 score MFMAs per tile
constexpr int kPvMfmas = 2 * kGroups * kCTiles;  // 32 output MFMAs per tile
constexpr int kLoadsPerWave = 9;       // 36 loads of 1 KiB per tile
constexpr int kStores = 2 * kGroups * kCTiles;   // epilogue: 16-byte stores per lane
constexpr float kTau = 8.0f;           // lazy-rescale threshold (log2 units)
constexpr int kXcds = 8;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] bits 3:0, vmcnt[5:4] bits
// 15:14, lgkmcnt bits 11:8), the other counters untouched.
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int lgkmcnt_imm(int n) { return 15 | (7 << 4) | (3 << 14) | (n << 8); }
// vector memory operations issued after an interval's first tile load: its 9
// tile loads and, when a piece's output was stored, 32 stores
constexpr int vm_after(int st) {
  const int n = kLoadsPerWave + st * kStores;
  return n > 63 ? 63 : n;
}

// Work-groups go to the dies round robin (work-group i to die i % 8); parts
// p of one die are contiguous, so the pieces of one request (neighbouring
// parts) mostly run on one die and share its L2 for their query rows.
__device__ __forceinline__ int part_of_block(int i, int parts) {
  const int x = i % kXcds, j = i / kXcds;
  const int per = parts / kXcds, extra = parts % kXcds;
  return x * per + min(x, extra) + j;
}

__device__ __forceinline__ uint32_t lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// An index-array entry the same for every lane, through the scalar cache.
__device__ __forceinline__ int32_t uniform_load(const int32_t* p, int64_t i) {
  using const_i32 = const __attribute__((address_space(4))) int32_t;
  return *((const_i32*)p + i);
}

__device__ __forceinline__ int page_count(int L) { return L > 0 ? (L + kPage - 1) / kPage : 0; }

__device__ __forceinline__ int chunk_swz(int k) {
  return 4 * ((k >> 1) & 1) + 2 * ((k >> 2) & 1) + ((k >> 4) & 1);
}

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

// A pointer the same in every lane, as a value the compiler sees as uniform
// (a buffer descriptor built from it then stays in scalar registers; from a
// value it takes for divergent, every buffer access is wrapped in a loop over
// the distinct descriptors).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ void mem_fence() { asm volatile("" ::: "memory"); }

// Work-group barrier without a memory fence of the compiler's (which would
// wait for every outstanding load, the tiles in flight included); callers
// wait for what the barrier must publish themselves.
__device__ __forceinline__ void barrier() {
  mem_fence();
  __builtin_amdgcn_s_barrier();
  mem_fence();
}

// An empty statement that claims to change x: values computed from x after it
// are not hoisted above it (out of the loop), where they would hold registers
// for the whole loop.
__device__ __forceinline__ uint32_t pinned(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
// Holds a computed value at this point of the instruction stream: the
// arithmetic that produces it cannot sink below (the compiler would otherwise
// move the softmax out of the MFMA slots it is placed in, down to where its
// results are stored).
__device__ __forceinline__ void hold(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void hold(uint32_t& x) { asm volatile("" : "+v"(x)); }

// This lane's index in its wave and its row and half, (n, h) = (lane % 32,
// lane / 32), read afresh where they are used: the id passes through pinned(),
// so nothing derived from it is kept live across the tile loop (at the
// register limit the compiler would spill such values and wait on all vector
// memory, the tile loads in flight included, to reload them).
struct Lane {
  uint32_t lane;
  int n, h;
};
__device__ __forceinline__ Lane lane_now() {
  const uint32_t l = pinned(lane_id());
  return {l, (int)(l & 31), (int)(l >> 5)};
}

// ---------------------------------------------------------------------------
// The part's tiles, in order.  Request b, with L_b keys, has pages
// [p0, p1) in the part (p0 = begin_page for the first request, p1 = end_page
// for the last) and tiles [2 p0, min(2 p1, ceil(L_b / 32))): the second half
// of a last page with at most 32 keys is no tile.  A piece is the tiles of
// one request in the part; the piece index of the first request is the
// plan's, the others' 0.
// ---------------------------------------------------------------------------
struct Part {
  int b_first, pg_first, b_last, pg_last, first_piece;
};

// A tile's request word: bits 0..19 the request (the host keeps bs below
// 2^20), bits 20..29 the keys of the request from the tile's first key on,
// capped at 1023 (enough: with at most 512 rows, a tile whose count reaches
// the cap has every key visible to every row), bit 30: the piece's first
// tile, bit 31: its last.
constexpr int kReqMask = (1 << 20) - 1;
constexpr int kRemShift = 20;
constexpr int kRemCap = 1023;
constexpr int kFirstBit = 1 << 30;
constexpr int kLastBit = (int)(1u << 31);

// Per-lane copies of request metadata, each read by one vector load: lane i
// holds the value of request b0 + i (0 past the array).  The tile loop reads
// them by v_readlane; a scalar load there would stall the wave for a memory
// round trip whenever it misses the scalar cache.  Requests past the
// 64-request window fall back to scalar loads.
struct ReqWin {
  int b0;
  int32_t v;
  const int32_t* src;
};
__device__ __forceinline__ ReqWin req_window(const int32_t* src, int n, int b0) {
  ReqWin w;
  w.b0 = b0;
  w.src = src;
  w.v = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(src), (short)0, 4 * n, 0x00020000),
      4u * (uint32_t)(b0 + (int)lane_id()), 0, 0);
  return w;
}
__device__ __forceinline__ int req_at(const ReqWin& w, int b) {
  const int i = b - w.b0;
  return (i >= 0 && i < 64) ? __builtin_amdgcn_readlane(w.v, i) : uniform_load(w.src, b);
}

__device__ __forceinline__ bool req_tiles(const Part& pt, const ReqWin& lens, int b, int& L,
                                          int& t0, int& t1) {
  L = req_at(lens, b);
  const int np = page_count(L);
  const int p0 = b == pt.b_first ? pt.pg_first : 0;
  const int p1 = b == pt.b_last ? min(pt.pg_last, np) : np;
  t0 = 2 * p0;
  t1 = min(2 * p1, (max(L, 0) + kTileKeys - 1) / kTileKeys);
  return t1 > t0;
}

__device__ __forceinline__ int count_tiles(const Part& pt, const ReqWin& lens) {
  int n = 0;
  for (int b = pt.b_first; b <= pt.b_last; ++b) {
    int L, t0, t1;
    if (req_tiles(pt, lens, b, L, t0, t1)) n += t1 - t0;
  }
  return n;
}

// Where the result of the piece of s goes: its partial slot (fp32 lse, bf16
// o) when the request has more than one piece, else the final output.
struct Dest {
  uint16_t* o;  // row 0 of the piece's 512-column rows
  float* lse;   // row 0 of its lse, or null
  int64_t valid;  // the slot exists (64 bits: no padding bytes)
};

__device__ __forceinline__ Dest piece_dest(int b, const Part& pt, const ReqWin& kbeg,
                                           uint16_t* partial_o, float* partial_lse,
                                           uint16_t* out, float* lse_out, const TileParams& P) {
  const int k0 = req_at(kbeg, b);
  const int k = req_at(kbeg, b + 1) - k0;
  const int piece = b == pt.b_first ? pt.first_piece : 0;
  Dest d;
  if (k > 1) {
    const int64_t slot = (int64_t)k0 + piece;
    d.valid = slot >= 0 && slot < P.partial_slots;
    d.o = partial_o + slot * P.rows * kDv;
    d.lse = partial_lse + slot * P.rows;
  } else {
    d.valid = 1;
    d.o = out + (int64_t)b * P.rows * kDv;
    d.lse = lse_out ? lse_out + (int64_t)b * P.rows : nullptr;
  }
  return d;
}

// ---------------------------------------------------------------------------
// Lane offsets (bytes, relative to a tile slot) of the MFMA operands.
//  * Score MFMA, A operand (K): lane (m = lane % 32, h = lane / 32) reads key
//    sigma(m) = 16 bit2(m) + 4 (m >> 3) + (m & 3), dims 16 ks + 8h .. +7, i.e.
//    column block ks / 4, 16-byte chunk 2 (ks % 4) + h.  With that key
//    order, lane (n, h) of the result holds the scores of row n for keys
//    16h + i, i = 0..15 (result register i).  Chunk 2i + h of a key is at
//    k_off ^ 32 i.
//  * Output MFMA, A operand (V^T) by ds_read_b64_tr_b16: in the 16-lane block
//    (h, c16) source lane s16 addresses key 16h + 8u + 4e + s16 / 4, columns
//    32 vt + 16 c16 + 4 (s16 % 4) .. +3; the block then holds column
//    32 vt + 16 c16 + s16 of keys 16h + 8u + 4e .. +3.  v_off is e = 0, u = 0,
//    vt even; vt odd is ^ 64, e = 1 is (+ 512) ^ 32, u = 1 is + 1024.  With the
//    weights of lane (n, h), keys 16h + 8u + j, as the B operand of k-step u,
//    the MFMA's key index 8h + j is key 16h + 8u + j of the tile in both.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t k_off(uint32_t lane) {
  const int n = lane & 31, h = lane >> 5;
  const int sig = 16 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
  return sig * 128 + ((h ^ chunk_swz(sig)) << 4);
}
__device__ __forceinline__ uint32_t v_off(uint32_t lane) {
  const int h = lane >> 5, s16 = lane & 15, c16 = (lane >> 4) & 1, a = s16 >> 2;
  const int cc = 2 * c16 + ((s16 >> 1) & 1);
  return (16 * h + a) * 128 + ((cc ^ (4 * (a >> 1) + h)) << 4) + 8 * (s16 & 1);
}
// Tile loads of wave w: key group w (keys 8w .. 8w+7), lane i to key
// 8w + i / 8, chunk slot i % 8, from source chunk (i % 8) ^ swz(8w + i / 8);
// column block k at immediate offset 128 k.
__device__ __forceinline__ uint32_t load_off(uint32_t lane, int w) {
  return (8 * w + (lane >> 3)) * kRowBytes +
         16 * ((lane & 7) ^ (4 * ((lane >> 4) & 1) + 2 * ((lane >> 5) & 1) + ((w >> 1) & 1)));
}

__device__ __forceinline__ uint32_t v_slot(int it) { return (uint32_t)(it & 3) * kVSlotBytes; }
__device__ __forceinline__ uint32_t rope_slot(int it) {
  return kRopeBase + (uint32_t)(it % kRopeSlots) * kBlockBytes;
}
__device__ __forceinline__ uint32_t p_buf(int it) { return kPBase + (uint32_t)(it & 1) * kPBufBytes; }
__device__ __forceinline__ uint32_t a_buf(int it) { return kABase + (uint32_t)(it & 1) * 512; }
__device__ __forceinline__ uint32_t i_buf(int it) { return kIBase + (uint32_t)(it & 1) * 512; }

// ---------------------------------------------------------------------------
// The chain of an interval, from inline assembly: one statement per MFMA or
// group of LDS reads, compiler scheduling barriers between statements, so the
// order written here is the order issued and every LDS read has its
// hand-placed lgkmcnt wait in front of the MFMA that reads it.  The LDS reads
// must be out of the compiler's sight: the wave also issues direct-to-LDS
// loads, and the compiler would make every LDS read it can see wait for all
// of them (vmcnt(0)).  A chain is straight-line code from its first read to
// its last MFMA, so nothing can move or copy a register whose read is still
// in flight.  Hazards the compiler cannot see: score MFMAs accumulate back to
// back into one register tile (an MFMA may read its predecessor's result as
// the accumulator); the softmax reads the scores after 24 wait states; an
// output tile is read by VALU code only after the chain's tail.
//
// Slots.  Variant kSP (scores of tile t and outputs of tile t-1): slots 0..35
// hold the 36 score MFMAs, slots 36..67 the 32 output MFMAs, with the softmax
// of tile t spread over them (it needs every score, and its arithmetic
// issues in the shadow of these output MFMAs).  kS: the 36 score MFMAs (the part's first tile);
// kP: the 32 output MFMAs (after the part's last tile).  Output MFMA m adds,
// for k-step u = m / 16, column tile c = (m % 16) / 4 and row group
// g = m % 4, V^T(c, u) P^T(g, u) to accumulator tile [g][c].
// Reads: key read k kAAhead score MFMAs ahead; the weights of the four row
// groups for u = 0 in the prologue, for u = 1 into the same registers after
// the last u = 0 use of each; the value operand (c, u) 3 slots before its
// first MFMA, into one of two sets.
// ---------------------------------------------------------------------------
enum { kSP = 0, kS = 1, kP = 2 };
constexpr int kAAhead = 6;
constexpr int kARing = kAAhead + 1;
constexpr int kHead = kKSteps;  // 36 slots of the score part of kSP
constexpr int kVLead = 3;   // value reads go out this many slots ahead

__host__ __device__ constexpr int n_slots(int var) {
  return var == kSP ? kKSteps + kPvMfmas : var == kS ? kKSteps : kPvMfmas;
}
__host__ __device__ constexpr bool is_pv(int var, int s) {
  return var == kS   ? false
         : var == kP ? true
                     : s >= kHead;
}
__host__ __device__ constexpr bool has_s(int var) { return var != kP; }
__host__ __device__ constexpr bool has_pv(int var) { return var != kS; }

// The schedule of a variant, worked out once at compile time.
constexpr int kMaxSlots = kKSteps + kPvMfmas;  // 68
struct Sched {
  int n;
  bool pv[kMaxSlots];        // slot holds an output MFMA
  int idx[kMaxSlots];        // score k-step or output MFMA index of the slot
  int slot_s[kKSteps];       // slot of score MFMA k
  int slot_o[kPvMfmas];      // slot of output MFMA m
  int pos_k[kKSteps];        // slot after which key read k goes out (-1: prologue)
  int pos_p[kGroups][2];     // weights of row group g, k-step u
  int pos_v[kCTiles][2];     // value operand of column tile c, k-step u (two reads)
  int seq_k[kKSteps];        // issue order of the LDS reads
  int seq_p[kGroups][2];
  int seq_v[kCTiles][2];     // (the second of the two)
  int wait[kMaxSlots];       // lgkmcnt before the MFMA of the slot
  bool ok;
};

__host__ __device__ constexpr Sched make_sched(int var) {
  Sched S{};
  S.n = n_slots(var);
  int ns = 0, no = 0;
  for (int s = 0; s < S.n; ++s) {
    const bool p = is_pv(var, s);
    S.pv[s] = p;
    S.idx[s] = p ? no : ns;
    if (p)
      S.slot_o[no++] = s;
    else
      S.slot_s[ns++] = s;
  }
  for (int k = 0; k < kKSteps; ++k)
    S.pos_k[k] = !has_s(var) ? -2 : k < kAAhead ? -1 : S.slot_s[k - kAAhead];
  for (int g = 0; g < kGroups; ++g)
    for (int u = 0; u < 2; ++u)
      // u = 1: into the u = 0 register, one slot after its last reader
      S.pos_p[g][u] = !has_pv(var) ? -2 : u == 0 ? -1 : S.slot_o[12 + g] + 1;
  for (int c = 0; c < kCTiles; ++c)
    for (int u = 0; u < 2; ++u) {
      const int x = has_pv(var) ? S.slot_o[16 * u + 4 * c] - kVLead : -2;
      S.pos_v[c][u] = !has_pv(var) ? -2 : x < -1 ? -1 : x;
    }
  // issue order at each position: key read, weights (u-major), value operands
  int seq = 0;
  int before[kMaxSlots + 1] = {};
  for (int x = -1; x < S.n; ++x) {
    for (int k = 0; k < kKSteps; ++k)
      if (S.pos_k[k] == x) S.seq_k[k] = seq++;
    for (int u = 0; u < 2; ++u)
      for (int g = 0; g < kGroups; ++g)
        if (S.pos_p[g][u] == x) S.seq_p[g][u] = seq++;
    for (int u = 0; u < 2; ++u)
      for (int c = 0; c < kCTiles; ++c)
        if (S.pos_v[c][u] == x) {
          seq += 2;
          S.seq_v[c][u] = seq - 1;
        }
    before[x + 1] = seq;  // reads issued before the MFMA of slot x + 1
  }
  S.ok = true;
  for (int s = 0; s < S.n; ++s) {
    int need;
    if (!S.pv[s]) {
      need = S.seq_k[S.idx[s]];
    } else {
      const int m = S.idx[s], u = m / 16, c = (m % 16) / 4, g = m % 4;
      need = S.seq_v[c][u] > S.seq_p[g][u] ? S.seq_v[c][u] : S.seq_p[g][u];
    }
    S.wait[s] = before[s] - need - 1;
    if (S.wait[s] < 0 || S.wait[s] > 15) S.ok = false;
  }
  if (has_pv(var)) {
    // a weights register is rewritten only after the last MFMA reading it
    // (and before the first of the next k-step), a value set only after the
    // last MFMA of the operand two before it
    for (int g = 0; g < kGroups; ++g)
      if (S.pos_p[g][1] <= S.slot_o[12 + g] || S.pos_p[g][1] >= S.slot_o[16 + g]) S.ok = false;
    for (int c = 0; c < kCTiles; ++c)
      for (int u = 0; u < 2; ++u) {
        const int prev = 16 * u + 4 * c - 8;  // same set, two operands before
        if (prev >= 0 && S.pos_v[c][u] <= S.slot_o[prev + 3]) S.ok = false;
      }
  }
  return S;
}

constexpr Sched kSchedSP = make_sched(kSP);
constexpr Sched kSchedS = make_sched(kS);
constexpr Sched kSchedP = make_sched(kP);
static_assert(kSchedSP.ok && kSchedS.ok && kSchedP.ok, "chain schedule");
static_assert(kSchedSP.slot_s[kKSteps - 1] < kHead, "scores before the softmax slots");

template <int VAR>
struct SchedOf;
template <>
struct SchedOf<kSP> {
  static constexpr const Sched& s = kSchedSP;
};
template <>
struct SchedOf<kS> {
  static constexpr const Sched& s = kSchedS;
};
template <>
struct SchedOf<kP> {
  static constexpr const Sched& s = kSchedP;
};

template <int N>
__device__ __forceinline__ void lgkm_wait() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(lgkmcnt_imm(N));
}

struct VOp {
  bf16x4 lo, hi;
};

// operands and accumulators of one chain
struct ChainRegs {
  bf16x8 kring[kARing];
  bf16x8 pw[kGroups];  // weights of the four row groups, current k-step
  VOp vs[2];           // value operands
};

struct ChainAddr {
  uint32_t ka[4];      // key reads: slot + (k_off ^ 32 i)
  uint32_t kr;         // rope slot - value slot (added for the rope reads)
  uint32_t va[2][2];   // value reads of tile t-1
  uint32_t pb;         // weights of tile t-1: p_buf + 16 lane
};

template <int K>
__device__ __forceinline__ void k_read(bf16x8& dst, const ChainAddr& A) {
  if constexpr (K < 32) {
    asm volatile("ds_read_b128 %0, %1 offset:%2"
                 : "=&v"(dst)
                 : "v"(A.ka[K & 3]), "i"(kBlockBytes * (K >> 2)));
  } else {
    uint32_t t;
    asm volatile("v_add_u32 %1, %3, %2\n\tds_read_b128 %0, %1"
                 : "=&v"(dst), "=&v"(t)
                 : "v"(A.ka[K & 3]), "s"(A.kr));
  }
}

template <int G, int U>
__device__ __forceinline__ void p_read(bf16x8& dst, const ChainAddr& A) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=&v"(dst) : "v"(A.pb), "i"(2048 * G + 1024 * U));
}

// value operand of column tile c (32 columns: tile vt = 4w + c of the value
// row, w the wave), k-step u
template <int C, int U>
__device__ __forceinline__ void v_read(VOp& o, const ChainAddr& A) {
  // vt = 4w + C: vt & 1 = C & 1 (4w even); vt >> 1 = 2w + C / 2 (the 2w part
  // is in va)
  constexpr int off = 1024 * U + kBlockBytes * (C >> 1);
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2 offset:%4\n\t"
      "ds_read_b64_tr_b16 %1, %3 offset:%4"
      : "=&v"(o.lo), "=&v"(o.hi)
      : "v"(A.va[0][C & 1]), "v"(A.va[1][C & 1]), "i"(off));
}

__device__ __forceinline__ bf16x8 cat(const VOp& v) {
  return __builtin_shufflevector(v.lo, v.hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// score MFMA (VGPR accumulator); ZERO starts the accumulation
template <bool ZERO>
__device__ __forceinline__ void mfma_s(f32x16& c, const bf16x8& a, const bf16x8& b) {
  if constexpr (ZERO)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// output MFMA (AGPR accumulator); ZERO: the tile's first terms of a piece
template <bool ZERO>
__device__ __forceinline__ void mfma_o(f32x16& o, const bf16x8& a, const bf16x8& b) {
  if constexpr (ZERO)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&a"(o) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
}

// The reads that go out after slot X (or the prologue, X = -1), in the
// order of the schedule: key read, weights, value operands.
template <int VAR, int X, int K>
__device__ __forceinline__ void k_read_if(ChainRegs& R, const ChainAddr& A) {
  if constexpr (SchedOf<VAR>::s.pos_k[K] == X) k_read<K>(R.kring[K % kARing], A);
}
template <int VAR, int X, int... K>
__device__ __forceinline__ void k_reads_at(std::integer_sequence<int, K...>, ChainRegs& R,
                                           const ChainAddr& A) {
  (k_read_if<VAR, X, K>(R, A), ...);
}
template <int VAR, int X, int G, int U>
__device__ __forceinline__ void p_read_if(ChainRegs& R, const ChainAddr& A) {
  if constexpr (SchedOf<VAR>::s.pos_p[G][U] == X) p_read<G, U>(R.pw[G], A);
}
template <int VAR, int X, int C, int U>
__device__ __forceinline__ void v_read_if(ChainRegs& R, const ChainAddr& A) {
  if constexpr (SchedOf<VAR>::s.pos_v[C][U] == X) v_read<C, U>(R.vs[C & 1], A);
}
template <int VAR, int X>
__device__ __forceinline__ void issue_reads(ChainRegs& R, const ChainAddr& A) {
  if constexpr (has_s(VAR)) k_reads_at<VAR, X>(std::make_integer_sequence<int, kKSteps>{}, R, A);
  if constexpr (has_pv(VAR)) {
    p_read_if<VAR, X, 0, 0>(R, A);
    p_read_if<VAR, X, 1, 0>(R, A);
    p_read_if<VAR, X, 2, 0>(R, A);
    p_read_if<VAR, X, 3, 0>(R, A);
    p_read_if<VAR, X, 0, 1>(R, A);
    p_read_if<VAR, X, 1, 1>(R, A);
    p_read_if<VAR, X, 2, 1>(R, A);
    p_read_if<VAR, X, 3, 1>(R, A);
    v_read_if<VAR, X, 0, 0>(R, A);
    v_read_if<VAR, X, 1, 0>(R, A);
    v_read_if<VAR, X, 2, 0>(R, A);
    v_read_if<VAR, X, 3, 0>(R, A);
    v_read_if<VAR, X, 0, 1>(R, A);
    v_read_if<VAR, X, 1, 1>(R, A);
    v_read_if<VAR, X, 2, 1>(R, A);
    v_read_if<VAR, X, 3, 1>(R, A);
  }
}

template <int N>
using ic = std::integral_constant<int, N>;

// Slot S: wait, MFMA, the reads that go out after it, then hook(ic<S>) (tile
// loads, query loads) and pay(ic<S>) (softmax arithmetic in the MFMA's shadow).
template <int VAR, bool PV_ZERO, int S, typename Hook, typename Pay>
__device__ __forceinline__ void slot(f32x16& s, f32x16 (&o)[kGroups][kCTiles], ChainRegs& R,
                                     const ChainAddr& A, const bf16x8 (&qreg)[kKSteps],
                                     Hook& hook, Pay& pay) {
  constexpr const Sched& SC = SchedOf<VAR>::s;
  lgkm_wait<SC.wait[S]>();
  SB();
  if constexpr (!SC.pv[S]) {
    constexpr int k = SC.idx[S];
    mfma_s<k == 0>(s, R.kring[k % kARing], qreg[k]);
  } else {
    constexpr int m = SC.idx[S], u = m / 16, c = (m % 16) / 4, g = m % 4;
    mfma_o<PV_ZERO && u == 0>(o[g][c], cat(R.vs[c & 1]), R.pw[g]);
  }
  SB();
  issue_reads<VAR, S>(R, A);
  SB();
  hook(ic<S>{});
  SB();
  pay(ic<S>{});
  SB();
}

template <int VAR, bool PV_ZERO, typename Hook, typename Pay, int... S>
__device__ __forceinline__ void slots(std::integer_sequence<int, S...>, f32x16& s,
                                      f32x16 (&o)[kGroups][kCTiles], ChainRegs& R,
                                      const ChainAddr& A, const bf16x8 (&qreg)[kKSteps],
                                      Hook& hook, Pay& pay) {
  (slot<VAR, PV_ZERO, S>(s, o, R, A, qreg, hook, pay), ...);
}

// The chain's slots; the caller has issued its first reads (issue_reads<VAR,
// -1>) into R.
template <int VAR, bool PV_ZERO, typename Hook, typename Pay>
__device__ __forceinline__ void chain(f32x16& s, f32x16 (&o)[kGroups][kCTiles], ChainRegs& R,
                                      const ChainAddr& A, const bf16x8 (&qreg)[kKSteps],
                                      Hook&& hook, Pay&& pay) {
  SB();
  slots<VAR, PV_ZERO>(std::make_integer_sequence<int, n_slots(VAR)>{}, s, o, R, A, qreg, hook,
                      pay);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");  // results of the last MFMAs
  SB();
}

// Multiply an accumulator tile (AGPRs) by alpha in place, through one VGPR.
// Written in assembly, element by element, so that the tile stays in AGPRs
// (the compiler would otherwise move all 256 accumulators to VGPRs and back
// for this rarely taken step).  The trailing wait states cover an MFMA that
// reads the tile next.
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
      : "+a"(e[0]), "+a"(e[1]), "+a"(e[2]), "+a"(e[3]), "+a"(e[4]), "+a"(e[5]), "+a"(e[6]),
        "+a"(e[7]), "+a"(e[8]), "+a"(e[9]), "+a"(e[10]), "+a"(e[11]), "+a"(e[12]),
        "+a"(e[13]), "+a"(e[14]), "+a"(e[15]), "=&v"(tmp)
      : "v"(alpha));
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = e[i];
}

// Stores accumulator tile `acc` (AGPRs) times `scale` as bf16.  The tile is
// O^T of 32 value columns x 32 rows: lane (n, h) holds row n, columns
// 8g + 4h + 0..3 in registers 4g .. 4g+3.  Groups 2q and 2q+1 are exchanged
// between the lane halves (v_permlane32_swap) so that each lane stores 8
// consecutive columns (16 bytes): columns 16q + 8h of the tile.  dst: the
// piece's rows as a buffer whose range ends with the last row that exists;
// off: the byte offset of the lane's row at the tile's first column.  Rows
// past the range are dropped by the hardware, so every lane issues both
// stores (the wait counts of the tile loads rely on a fixed number of store
// instructions).
__device__ __forceinline__ void store_tile(const f32x16& acc, float scale,
                                           __amdgpu_buffer_rsrc_t dst, uint32_t off, int h) {
  // the accumulators are read from assembly with AGPR operands, so the tile
  // stays in AGPRs (a plain copy lets the compiler move the tiles between
  // register files)
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[i]) : "a"(acc[i]));
#pragma unroll
  for (int qd = 0; qd < 2; ++qd) {
    const int g0 = 2 * qd, g1 = 2 * qd + 1;
    auto pk = [&](int i) __attribute__((always_inline)) {
      return __builtin_bit_cast(
          uint32_t, __builtin_convertvector((f32x2){v[i] * scale, v[i + 1] * scale}, bf16x2));
    };
    const uint32_t x0 = pk(4 * g0), x1 = pk(4 * g0 + 2);
    const uint32_t y0 = pk(4 * g1), y1 = pk(4 * g1 + 2);
    const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
    const u32x4 w = {s0[0], s1[0], s0[1], s1[1]};
    __builtin_amdgcn_raw_buffer_store_b128(w, dst, off + 2 * (16 * qd + 8 * h), 0, 0);
  }
}

// Clears the output accumulators with one MFMA per tile (zero operands, zero
// accumulator input): 16 instructions instead of 256 register writes.  The
// first one waits out the VALU write of the zero operand.
__device__ __forceinline__ void zero_acc(f32x16 (&o)[kGroups][kCTiles]) {
  const bf16x8 z = {};
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(o[0][0]) : "v"(z));
#pragma unroll
  for (int i = 1; i < kGroups * kCTiles; ++i)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(o[i / kCTiles][i % kCTiles]) : "v"(z));
}

struct TileLoad {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t vslot, rslot;  // LDS byte addresses of the destination slots
};

template <int K>
__device__ __forceinline__ void tile_load(const TileLoad& tl, int w, uint32_t voff) {
  // LDS address = M0 + immediate + 16 * lane: M0 is the destination minus the
  // immediate (the column block's offset in the source row)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      tl.rsrc, LDS_AT(void, (K < 8 ? tl.vslot + K * kBlockBytes : tl.rslot) + w * 1024 - K * 128),
      16, voff, 0, K * 128, /*nt*/ 2);
}

template <int... K>
__device__ __forceinline__ void tile_loads(std::integer_sequence<int, K...>, const TileLoad& tl,
                                           int w, uint32_t voff) {
  (tile_load<K>(tl, w, voff), ...);
}

// The slots after which the tile loads go out: every fourth score MFMA.
__host__ __device__ constexpr int load_at(int var, int s) {
  if (var == kSP || var == kS) return (s % 4 == 3 && s / 4 < kLoadsPerWave) ? s / 4 : -1;
  return -1;
}
static_assert(load_at(kSP, 35) == 8 && 35 < kHead && load_at(kS, 35) == 8,
              "9 tile loads per chain");

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <int VAR>
struct VarTag {};

__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_decode_tile_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
                       const int32_t* __restrict__ block_table,
                       const int32_t* __restrict__ seq_lens,
                       const int32_t* __restrict__ tile_plan,
                       const int32_t* __restrict__ split_indptr,
                       uint16_t* __restrict__ partial_o, float* __restrict__ partial_lse,
                       uint16_t* __restrict__ out, float* __restrict__ lse_out, TileParams P) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];
  const uint32_t smem_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = part_of_block(blockIdx.x, gridDim.x);

  const int32_t* tp = tile_plan + (int64_t)part * 8;
  Part pt;
  pt.b_first = uniform_load(tp, 0);
  pt.pg_first = uniform_load(tp, 1);
  pt.b_last = uniform_load(tp, 2);
  pt.pg_last = uniform_load(tp, 3);
  pt.first_piece = uniform_load(tp, 4);
  const int npages = uniform_load(tp, 5);
  // An empty part, or a row no planner writes, does nothing (uniform over the
  // work-group, before any barrier).
  if (npages <= 0 || pt.b_first < 0 || pt.b_last >= P.bs || pt.b_first > pt.b_last ||
      pt.pg_first < 0 || pt.pg_last < 0 || pt.first_piece < 0)
    return;
  // the lengths and first partial slots of the part's first 64 requests
  const ReqWin lens0 = req_window(seq_lens, P.bs, pt.b_first);
  const ReqWin kbeg = req_window(split_indptr, P.bs + 1, pt.b_first);
  const int T = count_tiles(pt, lens0);
  if (T <= 0) return;

  const int rb0 = blockIdx.y * kRowsPerBlock;  // the block's first row
  const int ws0 = rb0 + wave * kRowsPerWave;   // the wave's first score row
  const float c_log2 = fmaxf(P.scale_log2, 1e-30f);
  const int i_tok_min = min(ws0, P.rows - 1) / P.heads;

  // LDS starts as zeros: a load lane past a tile's range may leave its bytes
  // untouched, and the bytes the MFMAs read must be finite.
  for (int i = (int)threadIdx.x; i < kLdsBytes / 16; i += kThreads)
    *LDS_AT(u32x4, smem_base + 16 * i) = (u32x4){0, 0, 0, 0};
  __builtin_amdgcn_s_waitcnt(lgkmcnt_imm(0));
  barrier();

  // ---- the part's tiles, 64 at a time: lane j of the window describes tile
  // w0 + j of the part (the tiles in the order they run)
  //   w_tok: pool index of the tile's first key, page * 64 + 32 (t % 2), or -1
  //          when the block-table entry is outside the table or the pool (the
  //          tile then loads as zeros and all its keys are masked)
  //   w_bf:  its request word (request, remaining keys, first / last of piece)
  // The window is rebuilt when the tile loads reach its end (starting one
  // tile behind the score tile, so the four tiles in use stay inside).
  int32_t w_tok = -1, w_bf = 0;
  int w0 = 0;
  const int bt_bytes = 4 * P.bs * P.bt_stride;  // < 2^31: checked by the host
  auto load_window = [&](int base, const ReqWin& lens) __attribute__((always_inline)) {
    const int j = base + (int)lane_id();
    int bf = 0, addr = -1, half = 0, off = 0;
    for (int b = pt.b_first; b <= pt.b_last && off < base + 64; ++b) {
      int L, t0, t1;
      if (!req_tiles(pt, lens, b, L, t0, t1)) continue;
      const int nt = t1 - t0, k = j - off;
      if (k >= 0 && k < nt) {
        const int t = t0 + k;
        bf = b | (min(L - kTileKeys * t, kRemCap) << kRemShift) | (k == 0 ? kFirstBit : 0) |
             (k == nt - 1 ? kLastBit : 0);
        half = t & 1;
        addr = (t >> 1) < P.bt_stride ? b * P.bt_stride + (t >> 1) : -1;
      }
      off += nt;
    }
    const int32_t e = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(block_table), (short)0, bt_bytes,
                                          0x00020000),
        addr >= 0 ? 4u * (uint32_t)addr : 0x80000000u, 0, 0);
    w_tok = (addr >= 0 && e >= 0 && e < P.num_pages) ? e * kPage + half * kTileKeys : -1;
    w_bf = bf;
  };
  load_window(0, lens0);
  auto w_at = [&](int32_t v, int i) __attribute__((always_inline)) {
    return __builtin_amdgcn_readlane(v, i - w0);
  };

  // ---- tile loads: the descriptor of tile `it`'s loads (empty past the last tile)
  auto next_load = [&](int it) __attribute__((always_inline)) {
    TileLoad tl;
    const uint8_t* src = kv;
    int valid = 0;
    if (it < T) {
      const int tok = w_at(w_tok, it);
      if (tok >= 0) {
        src = kv + (int64_t)tok * kRowBytes;
        valid = min(kTileKeys, (w_at(w_bf, it) >> kRemShift) & kRemCap);
      }
    }
    src = uniform_ptr(src);
    valid = __builtin_amdgcn_readfirstlane(valid);
    tl.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), (short)0,
                                                valid * kRowBytes, 0x00020000);
    tl.vslot = smem_base + v_slot(it);
    tl.rslot = smem_base + rope_slot(it);
    return tl;
  };

  // ---- queries of the first piece, tiles 0 and 1
  bf16x8 qreg[kKSteps];
  // The queries of request b: one buffer over the request's rows, one lane
  // offset and 36 immediate offsets (rows past the last read as zeros).
  auto load_q = [&](int b) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(const_cast<uint16_t*>(q) + (int64_t)b * P.rows * kD), (short)0,
        P.rows * kD * (int)sizeof(uint16_t), 0x00020000);
    const Lane ln = lane_now();
    const uint32_t qoff = ((uint32_t)(ws0 + ln.n) * kD + 8 * ln.h) * 2;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qreg[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, qoff, 32 * ks, 0));
  };
  load_q(w_at(w_bf, 0) & kReqMask);
  {
    const uint32_t voff = load_off(lane_now().lane, wave);
    const TileLoad t0 = next_load(0);
    tile_loads(std::make_integer_sequence<int, kLoadsPerWave>{}, t0, wave, voff);
    const TileLoad t1 = next_load(1);
    tile_loads(std::make_integer_sequence<int, kLoadsPerWave>{}, t1, wave, voff);
  }
  // queries and tile 0 landed (tile 1's loads may still be in flight)
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerWave));
  barrier();

  f32x16 o[kGroups][kCTiles];
  float m_run = -INFINITY, l_run = 0.f;
  bool stored = false;    // this interval stored a piece's output

  // One interval: scores of tile `it` (it < T) and outputs of tile it-1
  // (it >= 1).  VAR: kS (the first tile), kSP, or kP (after the last tile).
  auto interval = [&](int it, auto var_tag) __attribute__((always_inline)) {
    constexpr int VAR = decltype(var_tag)::value;
    stored = false;
    const Lane ln = lane_now();
    const int n = ln.n, h = ln.h, r = ws0 + n;  // r: this lane's score row
    if (has_s(VAR) && it + 2 < T && it + 2 - w0 >= 64) {
      w0 = it - 1;  // rare: every 61 tiles
      load_window(w0, req_window(seq_lens, P.bs, pt.b_first));
    }
    // the output tile (it-1): the first of its piece starts from zero
    // accumulators
    const int pbf = has_pv(VAR) ? w_at(w_bf, it - 1) : 0;
    const bool o_first = has_pv(VAR) && (pbf & kFirstBit);
    const bool out_last = has_pv(VAR) && (pbf & kLastBit);
    if (o_first) zero_acc(o);
    // ---- the LDS reads go out first (the rescale factors of tile it-1, then
    // the chain's first operands); the interval's set-up runs in the shadow
    // of the first MFMAs
    ChainAddr A;
    const uint32_t vb = smem_base + v_slot(it);
#pragma unroll
    for (int i = 0; i < 4; ++i) A.ka[i] = vb + (k_off(ln.lane) ^ (32u * i));
    A.kr = __builtin_amdgcn_readfirstlane(smem_base + rope_slot(it) - vb);
    {
      const uint32_t vp = smem_base + v_slot(it - 1) + kBlockBytes * (2 * wave) + v_off(ln.lane);
      A.va[0][0] = vp;
      A.va[0][1] = vp ^ 64u;
      A.va[1][0] = (vp + 512u) ^ 32u;
      A.va[1][1] = A.va[1][0] ^ 64u;
    }
    A.pb = smem_base + p_buf(it - 1) + 16 * ln.lane;
    ChainRegs R;
    // the factors of the four row groups, [n][g] (older than every chain
    // read: the chain's first wait covers it)
    f32x4 al;
    SB();
    if constexpr (has_pv(VAR))
      asm volatile("ds_read_b128 %0, %1" : "=&v"(al) : "v"(smem_base + a_buf(it - 1) + 16 * n));
    SB();
    issue_reads<VAR, -1>(R, A);
    SB();
    // rescale the accumulators by the factors of tile it-1 (rows whose
    // running max moved) before its terms are added
    auto rescale = [&]() __attribute__((always_inline)) {
      if (!o_first &&
          __any(al[0] != 1.0f || al[1] != 1.0f || al[2] != 1.0f || al[3] != 1.0f)) {
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
#pragma unroll
          for (int c = 0; c < kCTiles; ++c) scale_tile(o[g][c], al[g]);
      }
    };
    if constexpr (VAR == kP) {
      // the first output MFMA is the chain's first: wait for the factors here
      lgkm_wait<0>();
      rescale();
    }
    // the score tile (it): its piece, its mask, the loads of tile it+2
    TileLoad tl{};
    int sbf = 0, vis = 16;
    bool s_first = false, s_last = false, more = false, defer = false;
    bool partial = false;  // some key of the tile is hidden from some row of the wave
    auto setup_s = [&]() __attribute__((always_inline)) {
      sbf = w_at(w_bf, it);
      s_first = sbf & kFirstBit;
      s_last = sbf & kLastBit;
      more = it + 1 < T;
      // at a piece's end the tile loads wait until the next piece's queries
      // have gone out (after the chain)
      defer = s_last && more;
      tl = next_load(it + 2);
    };
    auto setup_mask = [&]() __attribute__((always_inline)) {
      // last visible key of the wave's first row, relative to the tile's first key
      const int rem = (sbf >> kRemShift) & kRemCap;
      const int lim_min = P.causal ? rem - P.q_len + i_tok_min : rem - 1;
      const bool bad_page = w_at(w_tok, it) < 0;
      partial = bad_page || kTileKeys - 1 > lim_min;
      if (partial) {
        const int i_tok = r < P.rows ? r / P.heads : 0;
        const int lim = P.causal ? rem - P.q_len + i_tok : rem - 1;
        vis = bad_page ? 0 : min(16, lim - 16 * h + 1);
      }
      if (s_first) {
        m_run = -INFINITY;
        l_run = 0.f;
      }
    };
    const uint32_t voff = load_off(ln.lane, wave);
    f32x16 s;
    float ls = 0.f, alpha = 1.0f;
    uint32_t pk[8];
    auto hook = [&](auto sc) __attribute__((always_inline)) {
      constexpr int S = decltype(sc)::value;
      if constexpr (load_at(VAR, S) >= 0) {
        if (!defer) tile_load<load_at(VAR, S)>(tl, wave, voff);
      }
    };
    // the softmax of the score tile, in the shadow of the output MFMAs of the
    // tail slots kHead .. kHead+27 (kSP); after the chain for kS
    float mx = 0.f, m_tile = 0.f, neg_m = 0.f;
    auto soft = [&](auto step) __attribute__((always_inline)) {
      constexpr int k = decltype(step)::value;
      if constexpr (k == 0) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");  // the last score MFMA's result
        if (partial) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float x = i < vis ? s[i] : -INFINITY;
            hold(x);
            s[i] = x;
          }
        }
      } else if constexpr (k == 1) {
        mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                   fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
        hold(mx);
      } else if constexpr (k == 2) {
        mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])),
                             fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]))));
        m_tile = c_log2 * xhalf_max(mx);
        hold(m_tile);
      } else if constexpr (k == 3) {
        // lazy rescale: move the running max only when the tile's max exceeds
        // it by more than kTau (weights stay <= 2^kTau otherwise)
        const bool need = m_tile > m_run + kTau;
        const float m_new = need ? m_tile : m_run;
        alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        m_run = m_new;
        neg_m = m_run == -INFINITY ? 0.f : -m_run;  // -inf: no visible key yet
        hold(alpha);
        hold(m_run);
        hold(neg_m);
      } else if constexpr (k >= 4 && k < 12) {
        constexpr int i = 2 * (k - 4);
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[i], c_log2, neg_m));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[i + 1], c_log2, neg_m));
        ls += p0 + p1;
        pk[i >> 1] =
            __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0, p1}, bf16x2));
        hold(pk[i >> 1]);
        hold(ls);
      } else if constexpr (k == 12) {
        l_run = l_run * alpha + ls;
        hold(l_run);
      }
    };
    // the tail slot of each softmax step (kSP): the exponentials every third slot
    auto pay = [&](auto sc) __attribute__((always_inline)) {
      constexpr int X = decltype(sc)::value;
      if constexpr (X == 0 && has_s(VAR)) setup_s();
      if constexpr (X == 1 && VAR == kSP) rescale();  // before the first output MFMA
      if constexpr (X == 4 && has_s(VAR)) setup_mask();
      constexpr int S = X - kHead;
      if constexpr (VAR == kSP) {
        if constexpr (S == 0) soft(ic<0>{});
        if constexpr (S == 1) soft(ic<1>{});
        if constexpr (S == 2) soft(ic<2>{});
        if constexpr (S == 3) soft(ic<3>{});
        if constexpr (S >= 5 && S <= 26 && (S - 5) % 3 == 0) soft(ic<4 + (S - 5) / 3>{});
        if constexpr (S == 27) soft(ic<12>{});
      }
    };
    chain<VAR, false>(s, o, R, A, qreg, hook, pay);
    if constexpr (VAR == kS) {
      soft(ic<0>{});
      soft(ic<1>{}); soft(ic<2>{}); soft(ic<3>{}); soft(ic<4>{}); soft(ic<5>{});
      soft(ic<6>{}); soft(ic<7>{}); soft(ic<8>{}); soft(ic<9>{}); soft(ic<10>{});
      soft(ic<11>{}); soft(ic<12>{});
    }
    if constexpr (has_s(VAR)) {
      // ---- the next piece's queries (the score MFMAs have read these)
      if (s_last && more) {
        load_q(w_at(w_bf, it + 1) & kReqMask);
        // this interval's tile loads after the queries (kept in that order):
        // the wait for the next tile at the interval's end then covers the
        // queries too
        SB();
        tile_loads(std::make_integer_sequence<int, kLoadsPerWave>{}, tl, wave, voff);
      }
      // ---- hand the weights and the rescale factors to every wave
      // (LDS writes from assembly too: the compiler would make a write it
      // can see wait for the tile loads in flight; the barrier's lgkmcnt(0)
      // waits for them)
      const uint32_t pw = smem_base + p_buf(it) + 2048 * wave + 16 * ln.lane;
      const u32x4 w0 = {pk[0], pk[1], pk[2], pk[3]}, w1 = {pk[4], pk[5], pk[6], pk[7]};
      asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %2 offset:1024"
                   :
                   : "v"(pw), "v"(w0), "v"(w1)
                   : "memory");
      if (h == 0)
        asm volatile("ds_write_b32 %0, %1"
                     :
                     : "v"(smem_base + a_buf(it) + 16 * n + 4 * wave), "v"(alpha)
                     : "memory");
      if (s_last) {
        // ---- the score tile ends its piece: lse and the output scale
        const Dest ds = piece_dest(sbf & kReqMask, pt, kbeg, partial_o, partial_lse, out, lse_out, P);
        const float l_tot = xhalf_sum(l_run);
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        const float lse_val =
            l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
        if (h == 0)
          asm volatile("ds_write_b32 %0, %1"
                       :
                       : "v"(smem_base + i_buf(it) + 16 * n + 4 * wave), "v"(inv)
                       : "memory");
        if (ds.valid && h == 0 && ds.lse && r < P.rows) ds.lse[r] = lse_val;
      }
    }
    if constexpr (has_pv(VAR)) {
      // ---- the output tile ends its piece: store all 128 rows of this
      // wave's 128 columns
      const Dest d = out_last ? piece_dest(pbf & kReqMask, pt, kbeg, partial_o, partial_lse, out,
                                           lse_out, P)
                              : Dest{};
      if (out_last && d.valid) {
        f32x4 inv;
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                     : "=v"(inv)
                     : "v"(smem_base + i_buf(it - 1) + 16 * n));
        // the block's rows of the piece; the range ends with the request's last row
        const __amdgpu_buffer_rsrc_t dst = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(d.o + (int64_t)rb0 * kDv), (short)0, (P.rows - rb0) * kDv * (int)sizeof(uint16_t),
            0x00020000);
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
          const uint32_t roff = (uint32_t)(32 * g + n) * (kDv * 2);  // rows past the end: dropped
#pragma unroll
          for (int c = 0; c < kCTiles; ++c) {
            store_tile(o[g][c], inv[g], dst, roff + 64 * (4 * wave + c), h);
            SB();  // one tile's values in VGPRs at a time
          }
        }
        stored = true;
      }
    }
  };

  // The end of interval `it` (< T): tile it+1 and, at a piece's end, the next
  // queries landed (what was issued after them is this interval's 9 tile
  // loads and, when a piece ended, the 32 output stores), the weights,
  // factors and scales are in LDS; then the barrier.
  auto sync = [&]() __attribute__((always_inline)) {
    if (stored)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(vm_after(1)));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(vm_after(0)));
    __builtin_amdgcn_s_waitcnt(lgkmcnt_imm(0));
    barrier();
  };
  interval(0, ic<kS>{});
  sync();
  for (int it = 1; it < T; ++it) {
    interval(it, ic<kSP>{});
    sync();
  }
  interval(T, ic<kP>{});
  // every load has landed before the work-group's LDS is released
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

}  // namespace tile

mla_status launch_tile_decode(const void* q, const void* kv_cache, const int32_t* block_table,
                              const int32_t* seq_lens, const int32_t* tile_plan,
                              int32_t num_parts, const int32_t* split_indptr, void* partial_o,
                              float* partial_lse, void* out, float* lse, const TileParams& p,
                              hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  using namespace tile;
  const dim3 grid(num_parts, (unsigned)((p.rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(q);
  const uint8_t* kvp = reinterpret_cast<const uint8_t*>(kv_cache);
  uint16_t* po = reinterpret_cast<uint16_t*>(partial_o);
  uint16_t* op = reinterpret_cast<uint16_t*>(out);
  if (ev_start || ev_stop)
    hipExtLaunchKernelGGL(mla_decode_tile_kernel, grid, dim3(kThreads), 0, stream, ev_start,
                          ev_stop, 0, qp, kvp, block_table, seq_lens, tile_plan, split_indptr,
                          po, partial_lse, op, lse, p);
  else
    hipLaunchKernelGGL(mla_decode_tile_kernel, grid, dim3(kThreads), 0, stream, qp, kvp,
                       block_table, seq_lens, tile_plan, split_indptr, po, partial_lse, op, lse,
                       p);
  return check_launch("mla_decode");
}

}  // namespace mla
