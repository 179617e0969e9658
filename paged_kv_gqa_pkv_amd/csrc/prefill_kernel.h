// Causal chunked-prefill attention over a paged KV cache on bf16 MFMA, gfx950.
//
// What is computed (Module 12 page, model.py forward with T > 1: scores
// q K^T / sqrt(D) over the cached prefix plus the chunk, mask kpos <= qpos on
// absolute positions, softmax in fp32, probabilities times V; the chunk's
// K/V are appended before the call): for every query row of the chunk, the
// softmax-weighted sum of the V rows of its KV head over keys 0 .. its
// position.
//
// Decomposition.  The G = Hq/Hkv query heads of one KV head are stacked as
// extra rows (row R <-> token R / G, head R % G), so each K/V tile is used by
// all of them.  A workgroup of 4 waves owns 128 such rows of one (sequence,
// KV head) and one range of key tiles; each wave owns 32 rows.  Keys are
// walked in tiles of 64 (four pages, gathered through the block table) that
// the 4 waves share through LDS.  Tiles arrive by direct global->LDS loads
// (global_load_lds_dwordx4, one page per wave), so no registers hold data in
// flight: bf16 pages through separate K and V rings of two stages (64 KB,
// two workgroups per CU), int8 pages through a deeper ring of code stages.
// LDS rows are 256 B with their sixteen 16-byte chunks XOR-swizzled by row
// (one swizzle for K tiles, another for V tiles), which keeps the K reads
// (b128) and the V transpose reads free of bank conflicts without padding.
// When there are too few row tiles to fill the chip, the key range is cut
// into splits; each split writes its unnormalised (m, l, O), and the last
// split of a row tile to finish combines them in split order, in the same
// launch.
//
// The key loop is software-pipelined: the score products of tile i+1 run on
// the matrix cores while the VALU turns the scores of tile i into
// probabilities, and the PV products of tile i while tile i+1 is masked and
// its row max taken.  Exponentials and matrix products of one wave overlap;
// those of different waves on one SIMD mostly do not, so the overlap has to
// come from within the wave.
//
// Per tile and wave, on v_mfma_f32_32x32x16_bf16:
//   S^T[keys x rows] = K[keys x D] . Q^T[D x rows]   (2 key blocks x 8 k-steps)
//   O^T[D x rows]   += V^T[D x keys] . P^T[keys x rows] (4 dim blocks x 4 k-steps)
// Computing the transposed products puts one query row in each lane column,
// so the row max is a lane-local max plus one exchange with lane ^ 32, and
// the S^T accumulator registers are already the B operand of the PV product
// (the k index order inside an MFMA is free as long as both operands agree).
// The V^T operand comes straight from the row-major V tile through the LDS
// transpose read (ds_read_b64_tr_b16): in each 16-lane group, lane i receives
// element i%4 of the four 4-element rows addressed by lanes i/4 + 4k, so
// pointing lane j+4k at V[key_k][d0+4j] hands lane i the column
// V[key_0..3][d0+i].
// Softmax statistics stay in fp32; P is rounded to bf16 only as an MFMA
// operand, and the row sums use the same rounded values.  The running max is
// raised lazily (only when a row's max grows by more than 2^8), which keeps
// every exponent <= 2^8 and skips most accumulator rescales.
//
// int8 pages (Module 04 page, section 5, KV8Cache: a row is read back as
// its codes times its float32 scale).  The DMA ring then carries codes (half the bytes
// of a bf16 tile) and the pages' scale blocks; once a tile has landed, the
// workgroup dequantises it once into a bf16 tile (code * scale, rounded to
// bf16), double-buffered in LDS, and the MFMA work above runs unchanged on
// it.  Each element is converted once per workgroup, not once per wave.
//
// This header holds the device code (and the host-side argument packing)
// shared by the chunked-prefill launcher and the mixed-step launch.
#pragma once

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace pf {
namespace {


#ifndef PKV_PREFILL_WG_PER_CU
#define PKV_PREFILL_WG_PER_CU 1     // key-split planner: workgroups resident per CU
#endif
#ifndef PKV_PREFILL_MIN_TILES
#define PKV_PREFILL_MIN_TILES 2     // key-split planner: minimum tiles per split
#endif
#ifndef PKV_PREFILL_WG_COST_TILES
#define PKV_PREFILL_WG_COST_TILES 3   // planner: fixed workgroup cost, in tile-times
#endif
#ifndef PKV_PREFILL_MERGE_COST_TILES
#define PKV_PREFILL_MERGE_COST_TILES 3  // planner: split-merge cost, in tile-times
#endif

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerWG = kWaves * kRowsPerWave;   // 128
constexpr int kTileKeys = 64;                       // 4 pages
constexpr int kRowBytes = kD * 2;                   // 256 B per key row in LDS
constexpr int kTileBytes = kTileKeys * kRowBytes;   // 16 KB per K or V tile
#ifndef PKV_PREFILL_STAGES
#define PKV_PREFILL_STAGES 4        // int8 code ring depth (tiles in use: 2; loading: the rest)
#endif
constexpr int kStages = PKV_PREFILL_STAGES;
static_assert(kStages >= 3 && kStages <= 6, "two tiles in use plus at least one loading");
constexpr int kMaxTilesPerSplit = 64;               // page ids of a split fit in LDS
constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleSlack = 8.f;               // log2 units
constexpr int kMaxSplits = 32;                      // key splits per row tile (plan cap)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS layout.  Two bf16 K tiles, then two bf16 V tiles (bf16 pages: the
// two-stage K and V rings the DMA fills; int8 pages: the double-buffered
// dequantised tiles), then for int8 pages kStages code stages of {K codes,
// V codes, one 256 B scale DMA slot per page: the page's 16 K scales, then
// its 16 V scales, then a copy of both that is never read}.
constexpr int kCodeTileBytes = kTileKeys * kD;                 // 8 KB of codes
constexpr int kScaleSlotBytes = kWave * 4;                     // one 64-lane dword DMA
constexpr int kCodeStageBytes = 2 * kCodeTileBytes + 4 * kScaleSlotBytes;
template <bool kI8>
struct PrefillLds {
  static constexpr int kVOff = 2 * kTileBytes;
  static constexpr int kCodeOff = 4 * kTileBytes;
  static constexpr int kBytes = kI8 ? kCodeOff + kStages * kCodeStageBytes : 4 * kTileBytes;
  static constexpr int kVmPerTile = kI8 ? 5 : 4;   // DMA instructions per wave and tile (bf16: K or V)
};

struct PrefillArgs {
  uint16_t* out;                 // bf16 [total_q][Hq][D]
  const u32x4* q;                // bf16 [total_q][Hq][D] as 16-byte chunks
  const int32_t* cu_q;           // [B+1]
  const u32x4* k_cache;          // bf16 [num_blocks][16][Hkv][D], or int8 codes
  const u32x4* v_cache;
  const float* k_scales;         // int8 pages: float [num_blocks][Hkv][16]
  const float* v_scales;
  const int32_t* block_tables;   // [B][max_blocks]
  const int32_t* ctx_lens;       // [B]
  // Chunk rows taken from the step's new rows (bf16 pages, no ring; the
  // prefill body's kFresh instance): positions n - T .. n - 1 of sequence b (its chunk) are read
  // from rows cu_q[b] .. cu_q[b] + T - 1 of k_new / v_new ([total_q][Hkv][D],
  // the same row stride as a page) instead of the pool, whose slots for them
  // are written by others during the same launch.
  const u32x4* k_new;
  const u32x4* v_new;
  float* ws_acc;                 // [groups][splits][D/4][128 rows][4]
  float* ws_ml;                  // [groups][splits][128 rows][2]
  int* counters;                 // [groups] arrivals of the group's splits
  int B, total_q, max_q_len, Hq, Hkv, G, num_blocks, max_blocks, qtiles, splits,
      tiles_per_split;
  int window;                    // > 0: the pages form a ring of `window` tokens
  int neg_q;                     // scale < 0: q enters with its sign flipped
  float scale_log2;              // |scale| * log2(e), > 0
};

// Chunk swizzles of the LDS key rows: logical 16-byte chunk c of row r sits at
// position c ^ sw(r).  Both keep chunk pairs (2m, 2m+1) together and give
// rows 0..15 sixteen distinct values, so a 16-lane group of b128 reads (one
// row each) or of DMA writes (one row) covers all banks.
//  - K tiles, swz: the b128 K reads take rows 0..15 in one 16-lane group.
//  - V tiles, swzv: a b64 transpose read serves lanes 0..31 in one cycle and
//    32..63 in the next, and each half reads 4 rows (r & 3 = 0..3) in one
//    4-chunk group of dims.  swzv puts r & 3 in chunk bits 2-3, so the 4 rows
//    land in 4 different groups and each half covers all 256 bytes of banks.
//    (With swz the halves reached only chunks 0..7 or 8..15: two cycles more
//    per read, as the LDS bank-conflict counter showed.)
__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int swzv(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Direct global->LDS copy of 16 bytes per lane: lane i writes LDS bytes
// [lds + 16 i, lds + 16 i + 16).  Issued as inline asm so that the compiler
// does not wait for it before unrelated LDS reads; completion is awaited
// explicitly with s_waitcnt vmcnt before the tile is read.  The asm sets m0
// (the LDS base of the copy) without declaring it: the compiler reserves m0
// (it refuses it as a clobber) and nothing else in these kernels reads it
// (LDS instructions on gfx9 and later do not use it).
__device__ __forceinline__ void dma16(const u32x4* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(lds) : "memory");
}
// The same from a uniform base (SGPRs) plus a 32-bit per-lane byte offset:
// the address costs no vector instructions when only the base changes from
// one page to the next.
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(lds) : "memory");
}
// The same with 4 bytes per lane: lane i writes LDS bytes [lds + 4 i, lds + 4 i + 4).
__device__ __forceinline__ void dma4(const float* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(lds) : "memory");
}

// Split partials are written with agent-coherent stores: the last split of a
// group to finish, possibly on another XCD, reads them back.
__device__ __forceinline__ void ws_store(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
// Buffer loads of the split partials: the descriptor's last word for
// untyped 32-bit data on this architecture family, and the cache-policy
// operand of an agent-coherent access (sc1: read past the non-coherent
// caches, as the agent-scope stores wrote past them).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kCoherent = 16;

// 16 bytes per lane with the same coherence (the store instruction the
// agent-scope atomic store above compiles to, for four floats).  The s_nop
// is the wait state a store of more than 8 bytes needs before its data
// registers may be overwritten, which the compiler does not insert after
// inline asm.
__device__ __forceinline__ void ws_store4(float* p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 0" :: "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void ws_store2(float* p, float lo, float hi) {
  const uint64_t bits = (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), bits, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// 32-bit LDS byte offset of a __shared__ object.
__device__ __forceinline__ uint32_t lds_offset(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// s_waitcnt immediate: vector-memory count n, export and LDS counts left open.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Wait until the DMA loads of at most `ahead` later tiles (0 .. 3) of this
// wave are still in flight, P loads per tile.
template <int P>
__device__ __forceinline__ void wait_tiles(int ahead) {
  if (ahead >= 3)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * P));
  else if (ahead == 2)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * P));
  else if (ahead == 1)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(P));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// max of three floats in one instruction.  Written out because fmaxf on
// MFMA results costs an extra NaN-quieting max per operand (the compiler
// cannot tell they are canonical).
template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// The rows of sequence b and the keys that row tile x of them needs, and how
// many key splits hold some of them.
struct TileKeys {
  int q_lo, T, n;
  bool skip;          // rows outside [0, total_q), more than max_q_len, or none in this tile
  bool bad_len;       // more rows than context (or than the ring): NaN rows
  int key_lo, key_end, tile_first, n_tiles, ns;   // ns: non-empty key splits
};

__device__ __forceinline__ TileKeys tile_keys(const PrefillArgs& a, int b, int x) {
  TileKeys k;
  k.q_lo = a.cu_q[b];
  k.T = a.cu_q[b + 1] - k.q_lo;
  k.n = a.ctx_lens[b];
  const int R0 = x * kRowsPerWG;
  k.skip = k.q_lo < 0 || k.T < 0 || k.q_lo + k.T > a.total_q || k.T > a.max_q_len ||
           R0 >= k.T * a.G;
  // Ring paging (Module 04 page, section 4): position p sits at ring index
  // p % window, i.e. in the table's page (p / 16) % (window / 16); the ring
  // holds positions n - window .. n - 1, so keys below key_lo are gone.
  const bool ring = a.window > 0;
  bool bad = k.T > k.n || (ring ? k.T > a.window : k.n > a.max_blocks * kPage);
  // A context with more key tiles than the launch covers (a length past the
  // host's max_context_len) poisons the sequence's rows, as in decode, rather
  // than dropping the keys no split reaches.
  const int seq_key_lo = ring ? max(0, k.n - a.window) : 0;
  const int seq_tiles = (k.n + kTileKeys - 1) / kTileKeys - seq_key_lo / kTileKeys;
  bad = bad || seq_tiles > a.splits * a.tiles_per_split;
  k.bad_len = bad;
  // Keys: 0 .. the last position of the tile's rows (from key_lo in a ring).
  const int t_last = min(k.T - 1, (R0 + kRowsPerWG - 1) / a.G);
  k.key_end = bad ? 0 : k.n - k.T + t_last + 1;
  k.key_lo = bad ? 0 : seq_key_lo;
  k.tile_first = k.key_lo / kTileKeys;
  const int tile_end = (k.key_end + kTileKeys - 1) / kTileKeys;
  k.n_tiles = max(0, tile_end - k.tile_first);
  k.ns = (k.n_tiles + a.tiles_per_split - 1) / a.tiles_per_split;
  return k;
}

// The workgroup of block bid (see the grid order below).
template <bool kI8, bool kFresh = false>
__device__ __forceinline__ void prefill_body(const PrefillArgs a, const int bid) {
  using Lds = PrefillLds<kI8>;
  __shared__ __attribute__((aligned(1024))) char smem[Lds::kBytes];
  __shared__ int s_ids[kMaxTilesPerSplit * 4];
  __shared__ int s_bad, s_last;

  // ((b * qtiles + x) * splits + ks) * Hkv + g: the KV head varies fastest, so
  // all workgroups of KV head g land on XCD g % 8 and share its L2.
  const int g = bid % a.Hkv;
  int rest = bid / a.Hkv;
  const int ks = rest % a.splits;
  rest /= a.splits;
  const int x = a.qtiles - 1 - (rest % a.qtiles);   // heaviest (latest) row tiles first
  const int b = rest / a.qtiles;
  const int group = (b * a.qtiles + x) * a.Hkv + g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int G = a.G;

  // Rows outside [0, total_q) or more than max_q_len of them: nothing is read
  // or written for this sequence (its rows, if any exist, are not ours).
  const TileKeys tk = tile_keys(a, b, x);
  if (tk.skip) return;                        // uniform over the workgroup
  const int q_lo = tk.q_lo, T = tk.T, n = tk.n;
  const int R0 = x * kRowsPerWG;
  const bool ring = a.window > 0;
  const int ring_pages = ring ? a.window / kPage : 0;
  const bool bad_len = tk.bad_len;

  // This lane's query row (lane column of the MFMA tiles).
  const int row = R0 + w * kRowsPerWave + (lane & 31);
  const int t_row = row / G, j_row = row % G;
  const bool row_ok = t_row < T;
  const int qpos = row_ok ? n - T + t_row : -1;
  const int half = lane >> 5;                 // which 8 of 16 k values the lane holds

  // This split's share of the key tiles.
  const int key_end = tk.key_end, key_lo = tk.key_lo;
  const int tile_end = tk.tile_first + tk.n_tiles;
  const int tile0 = tk.tile_first + ks * a.tiles_per_split;
  const int tile1 = min(tile0 + a.tiles_per_split, tile_end);
  if (tile0 >= tile1) {
    if (ks == 0 && row_ok) {                  // bad length: no keys at all -> NaN rows
      uint32_t* orow = reinterpret_cast<uint32_t*>(
          a.out + ((int64_t)(q_lo + t_row) * a.Hq + g * G + j_row) * kD);
      for (int i = half; i < kD / 2; i += 2) orow[i] = 0x7fc07fc0u;
    }
    return;
  }
  const int nt = tile1 - tile0;               // <= kMaxTilesPerSplit by the plan
  const int qpos_min = n - T + R0 / G;        // smallest position in the workgroup
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;

  // Q^T as the B operand: lane holds Q[row][16kk + 8*half .. +8], kk = 0..7.
  bf16x8 qb[8];
  {
    const u32x4* qp = a.q + ((int64_t)(q_lo + t_row) * a.Hq + g * G + j_row) * 16;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok && !bad_len) v = qp[2 * kk + half];
      if (a.neg_q) v ^= 0x80008000u;          // (-q) . k * |scale| = q . k * scale, exactly
      qb[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Page ids of this split's tiles into LDS (0 for pages the workgroup does
  // not need); invalid ids of needed pages poison the result.
  int bad = 0;
  for (int p = tid; p < nt * 4; p += kWaves * kWave) {
    const int page = tile0 * 4 + p;             // page of absolute positions
    const int tpage = ring ? page % ring_pages : page;
    int id = 0;
    if (page * kPage < key_end && page * kPage + kPage > key_lo && tpage < a.max_blocks) {
      id = bt[tpage];
      if (id < 0 || id >= a.num_blocks) { bad = 1; id = 0; }
    }
    s_ids[p] = id;
  }

  // The ring's DMA loads are invisible to the compiler's wait counting, so
  // if a plain load (Q, the table) could still be in flight when the loop
  // starts, it would wait for vmcnt(0), i.e. for every tile in flight,
  // before each tile's first MFMA.  One explicit full wait here (Q has been
  // loading during the table reads) keeps those waits out of the loop.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  // Lane t of this wave holds the id of the wave's page of tile t (nt <= 64),
  // so that a step takes its page ids with readlane instead of LDS reads.
  const int wave_ids = lane < nt ? s_ids[4 * lane + w] : 0;

  // DMA of tile i (relative): wave w copies page w of the tile, the 16 rows
  // of KV head g (token-major pages: Hkv rows apart).  bf16: the K or the V
  // rows into stage i % 2 of their ring, 4 instructions of 4 rows; lane l of
  // instruction q fills row 16w + 4q + l/16 at chunk position l%16 with
  // logical chunk (l%16) ^ sw(row).  int8: the page's 16 rows of 128 K codes
  // and of V codes (2 instructions each, 8 rows per instruction, written in
  // row order 128 B apart) and its scales (one dword instruction: lanes 0..15
  // the K scales of slots 0..15, lanes 16..31 the V scales, lanes 32..63 the
  // same again into bytes that are never read).
  const uint32_t k_lds = lds_offset(smem);
  const uint32_t v_lds = k_lds + Lds::kVOff;
  const int dma_r16 = lane >> 4;              // + 4q: row within the page
  // Byte offsets of this lane's 16-byte piece within a page (bf16: row
  // r16 = 4q + lane/16 of head g, chunk (lane%16) ^ swizzle, per DMA
  // instruction q and K or V; int8: row 8q + lane/8, chunk lane%8), and the
  // bytes of one page of the pool.
  uint32_t koff[kI8 ? 2 : 4], voff[kI8 ? 1 : 4];
  if constexpr (kI8) {
#pragma unroll
    for (int qd = 0; qd < 2; ++qd)
      koff[qd] = (uint32_t)((((8 * qd + (lane >> 3)) * a.Hkv + g) * 8 + (lane & 7)) * 16);
    voff[0] = 0;
  } else {
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int r16 = 4 * qd + dma_r16;
      koff[qd] = (uint32_t)(((r16 * a.Hkv + g) * 16 + ((lane & 15) ^ swz(r16))) * 16);
      voff[qd] = (uint32_t)(((r16 * a.Hkv + g) * 16 + ((lane & 15) ^ swzv(r16))) * 16);
    }
  }
  const int64_t page_bytes = (int64_t)kPage * a.Hkv * kD * (kI8 ? 1 : 2);
  auto issue = [&](int i, bool is_v = false) {
    const int stage = kI8 ? i % kStages : (i & 1);
    const int64_t blk = __builtin_amdgcn_readlane(wave_ids, i);
    if constexpr (kI8) {
      (void)is_v;
      const uint32_t cs = k_lds + Lds::kCodeOff + stage * kCodeStageBytes;
      const char* kb = reinterpret_cast<const char*>(a.k_cache) + blk * page_bytes;
      const char* vb = reinterpret_cast<const char*>(a.v_cache) + blk * page_bytes;
#pragma unroll
      for (int qd = 0; qd < 2; ++qd) {
        const uint32_t off = (uint32_t)(w * kPage * kD + qd * 1024);
        dma16s(kb, koff[qd], cs + off);
        dma16s(vb, koff[qd], cs + kCodeTileBytes + off);
      }
      const int si = lane & 31;
      dma4(((si & 16) ? a.v_scales : a.k_scales) + (blk * a.Hkv + g) * kPage + (si & 15),
           cs + 2 * kCodeTileBytes + w * kScaleSlotBytes);
    } else {
      const uint32_t lds0 = (is_v ? v_lds : k_lds) + stage * kTileBytes + 16 * w * kRowBytes;
      const char* base = reinterpret_cast<const char*>(is_v ? a.v_cache : a.k_cache) +
                         blk * page_bytes;
      if constexpr (kFresh) {
        // Chunk rows from k_new / v_new: positions n - T .. n - 1 come from
        // there.  A page wholly inside them is one base (the new rows have a
        // page's row stride); a page that straddles either end of them
        // picks its source per lane.
        const int pos0 = ((tile0 + i) * 4 + w) * kPage;
        const int f0 = n - T;
        if (pos0 >= f0 && pos0 + kPage <= n) {
          base = reinterpret_cast<const char*>(is_v ? a.v_new : a.k_new) +
                 (int64_t)(q_lo + pos0 - f0) * a.Hkv * kRowBytes;
        } else if (pos0 + kPage > f0 && pos0 < n) {
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const int r16 = 4 * qd + dma_r16;
            const int c = (lane & 15) ^ (is_v ? swzv(r16) : swz(r16));
            const int pos = pos0 + r16;
            const bool fresh = pos >= f0 && pos < n;
            const int64_t idx = fresh ? ((int64_t)(q_lo + pos - f0) * a.Hkv + g) * 16 + c
                                      : ((blk * kPage + r16) * a.Hkv + g) * 16 + c;
            const u32x4* src =
                (is_v ? (fresh ? a.v_new : a.v_cache) : (fresh ? a.k_new : a.k_cache)) + idx;
            dma16(src, lds0 + 4 * qd * kRowBytes);
          }
          return;
        }
      }
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        dma16s(base, is_v ? voff[qd] : koff[qd], lds0 + 4 * qd * kRowBytes);
    }
  };

  // int8: dequantise the K (which = 0) or V (which = 1) codes of code stage
  // `stage` into bf16 buffer `buf` of that kind (swizzled rows, as the bf16
  // DMA writes them).  Thread: rows tid/8 and tid/8 + 32, 16 codes (dims
  // 16c .. 16c+15, c = tid % 8).  V rows outside [key_lo, key_end) get
  // scale 0: they are never visible, and zeros keep whatever their slots
  // hold out of the PV product.
  auto dequant = [&](int stage, int buf, int which, int key0) {
    const char* cs = smem + Lds::kCodeOff + stage * kCodeStageBytes;
    const int c = tid & 7;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = (tid >> 3) + 32 * k;         // key row of the tile
      const u32x4 cw = *reinterpret_cast<const u32x4*>(cs + which * kCodeTileBytes + r * kD + c * 16);
      const int slot = r & 15;                   // scales of a page: 16 K, then 16 V
      float sc = *reinterpret_cast<const float*>(
          cs + 2 * kCodeTileBytes + (r >> 4) * kScaleSlotBytes + (which * 16 + slot) * 4);
      if (which && (key0 + r >= key_end || key0 + r < key_lo)) sc = 0.f;
      uint32_t o8[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o8[2 * j] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)(sbyte0(cw[j]) * sc),
                                                        (__bf16)(sbyte1(cw[j]) * sc)});
        o8[2 * j + 1] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)(sbyte2(cw[j]) * sc),
                                                            (__bf16)(sbyte3(cw[j]) * sc)});
      }
      char* dst = smem + which * Lds::kVOff + buf * kTileBytes + r * kRowBytes;
      const int sw = which ? swzv(r) : swz(r);
      *reinterpret_cast<u32x4*>(dst + (((2 * c) ^ sw) << 4)) = u32x4{o8[0], o8[1], o8[2], o8[3]};
      *reinterpret_cast<u32x4*>(dst + (((2 * c + 1) ^ sw) << 4)) =
          u32x4{o8[4], o8[5], o8[6], o8[7]};
    }
  };

  // Lane read offsets.  K (A operand of S^T): row r = lane%32 (+32 per key
  // block), logical chunk 2kk + half, i.e. byte r*256 + ((2kk + half) ^
  // swz(r))*16 = kbase ^ 32kk.  V (transpose reads): row r = 8p + 4half + m/4
  // (+32kb + 16hh), dims 32db + 16*(lane/16 % 2) + 4*(m%4), i.e. logical
  // chunk c = 4db + 2*(lane/16 % 2) + (m%4)/2 at byte r*256 + (c ^ swzv(r))*16
  // + 8*(m%2) = vbase[p] ^ 64db.  (The XOR terms sit in bits 4-7, clear of
  // the row and stage bits, so a stage offset can be added first.)  One
  // register per base instead of one per offset keeps the kernel within the
  // two-waves-per-SIMD register budget.
  const int kbase = (lane & 31) * kRowBytes + ((half ^ swz(lane & 31)) << 4);
  int vbase[2];
  {
    const int m = lane & 15, k4 = m >> 2, j = m & 3, dh = (lane >> 4) & 1;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = 8 * p + 4 * half + k4;
      vbase[p] = r * kRowBytes + (((2 * dh + (j >> 1)) ^ swzv(r)) << 4) + (j & 1) * 8;
    }
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m = kNegInf, l = 0.f;

  // Software pipeline over the key tiles.  Step i, one wave's view:
  //   phase A: S(i+1) = K(i+1) Q^T on the matrix cores while the VALU turns
  //            S(i) into probabilities P(i);
  //   phase B: O += V(i)^T P(i) on the matrix cores while S(i+1) is masked
  //            (tiles on the diagonal or the ring's lower bound) and its row
  //            max taken; the max is raised (O and l rescaled) after the PV
  //            products.
  // Every tile still goes mask -> max -> raise -> probabilities -> products,
  // and O sees the products and rescales in tile order, so the result is
  // the one of processing the tiles one at a time.  The score products of
  // the next tile and the probabilities of this one are independent, which
  // keeps the matrix cores fed from one wave.
  //
  // Loads.  bf16 pages: separate K and V rings of two stages (64 KB, two
  // workgroups per CU); step i reads K(i+1) and V(i) while K(i+2) and
  // V(i+1) load.  int8 pages: one ring of kStages code stages, each tile
  // dequantised (K and V) into one of two bf16 buffers one step ahead.
  auto key0_of = [&](int i) { return (tile0 + i) * kTileKeys; };
  auto needs_mask = [&](int i) {
    const int key0 = key0_of(i);
    return key0 + kTileKeys - 1 > qpos_min || key0 < key_lo;
  };
  // Tiles with keys outside [key_lo, key_end): their V rows are zeroed.
  auto has_invisible = [&](int i) {
    const int key0 = key0_of(i);
    return key0 + kTileKeys > key_end || key0 < key_lo;
  };
  // LDS byte offsets of the K and V tiles of tile i, passed through an
  // empty asm so that the read addresses are formed inside each step (the
  // loop is unrolled by two, which would otherwise make all 16 of them
  // loop-invariant and keep them in registers).
  auto k_tile = [&](int i) {
    int off = (i & 1) * kTileBytes + kbase;
    asm volatile("" : "+v"(off));
    return off;
  };
  auto v_tile = [&](int i) {
    int off = Lds::kVOff + (i & 1) * kTileBytes;
    asm volatile("" : "+s"(off));
    return off;
  };

  // int8 pages: step i reads the bf16 K(i+1) and V(i) and, between its two
  // phases, dequantises K(i+2) and V(i+1) into the buffers of K(i) and
  // V(i-1), which every wave finished with before the step's barrier; the
  // barrier at the top of step i+1 publishes them.  So the codes of tile j
  // are read in steps j - 2 (K) and j - 1 (V), and the code ring holds tiles
  // i+1 .. i + kStages during step i: tile i + kStages is issued at the top
  // of step i into the stage of tile i.  Called only in steps with a next
  // tile; in the one before the last, K(i+2) does not exist and the call
  // turns stale codes into a buffer that is never read again (no branch, so
  // that the dequantisation stays in one scheduling region with the PV
  // products).
  auto dequant_ahead = [&](int i) {
    dequant((i + 2) % kStages, i & 1, 0, key0_of(i + 2));
    dequant((i + 1) % kStages, (i + 1) & 1, 1, key0_of(i + 1));
  };
  // Before step i: K(i+1) (if any) and V(i) become readable everywhere.
  auto top = [&](int i) {
    if constexpr (kI8) {
      // the codes of tile i+2, issued before step i - 1 or in the prologue
      if (i + 2 < nt) wait_tiles<Lds::kVmPerTile>(min(kStages - 3, nt - 3 - i));
      __syncthreads();
      if (i + kStages < nt) issue(i + kStages);
    } else {
      // K(i+1) and V(i), issued before step i - 1, are the only loads in
      // flight; after the barrier every wave is done with step i - 1, so
      // K(i)'s and V(i-1)'s stages take K(i+2) and V(i+1).
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
      if (i + 2 < nt) issue(i + 2, false);
      if (i + 1 < nt) issue(i + 1, true);
      if (has_invisible(i)) {
        // Keys past key_end (and, in a ring, below key_lo) are always
        // masked; zero their V rows so the canary NaNs of unwritten slots
        // cannot reach the products (K is masked).
        char* vz = smem + Lds::kVOff + (i & 1) * kTileBytes;
        const int key0 = key0_of(i);
        const u32x4 zero = {0u, 0u, 0u, 0u};
        for (int e = tid; e < kTileKeys * 16; e += kWaves * kWave) {
          const int r = e >> 4;
          if (key0 + r >= key_end || key0 + r < key_lo)
            *reinterpret_cast<u32x4*>(vz + r * kRowBytes + (e & 15) * 16) = zero;
        }
        __syncthreads();
      }
    }
  };

  // S^T = K . Q^T for the two 32-key blocks of a tile.
  auto scores = [&](f32x16 (&s)[2], int kof) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) s[kb][ii] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(smem + ((kof ^ (kk << 5)) + kb * 32 * kRowBytes));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[kk], s[kb], 0, 0, 0);
      }
    }
  };
  // Causal mask (and the ring's lower bound) in place; accumulator ii of
  // block kb holds key key0 + 32*kb + 8*(ii/4) + 4*half + ii%4.
  auto mask = [&](f32x16 (&s)[2], int key0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        const int key = key0 + 32 * kb + 8 * (ii >> 2) + 4 * half + (ii & 3);
        s[kb][ii] = (key <= qpos && key >= key_lo) ? s[kb][ii] : kNegInf;
      }
  };
  // Row max of a tile, scaled.
  auto tile_max = [&](const f32x16 (&s)[2]) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ii = 0; ii < 16; ii += 2) mx = max3(mx, s[kb][ii], s[kb][ii + 1]);
    const Halves h = halves32(mx);
    return max3(h.lo, h.hi, h.hi) * a.scale_log2;
  };
  // Raise the running max only when it grows by more than the slack (or on
  // the first visible key); exponents stay <= 2^slack.
  auto raise_max = [&](float mx) {
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack) == 0) return;
    const float m_new = fmaxf(m, mx);
    const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) o[db][ii] *= alpha;
  };
  // P^T of a tile in bf16, two values per convert, exp2(s * scale_log2 - m)
  // with one fma per score (scale > 0; m in the scaled domain): the B
  // operand of the PV product, k-step (kb, hh) = registers 8*hh .. 8*hh+7 of
  // block kb.  The row sum adds the same rounded values, a pair per v_dot2
  // with (1, 1), and is added to l.
  bf16x8 pb[2][2];
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  auto probs = [&](const f32x16 (&s)[2]) {
    const float nmu = (m == kNegInf) ? 0.f : -m;
    float lp[2] = {0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ii = 8 * hh + 2 * e;
          const bf16x2 pp = {(__bf16)fast_exp2(__builtin_fmaf(s[kb][ii], a.scale_log2, nmu)),
                             (__bf16)fast_exp2(__builtin_fmaf(s[kb][ii + 1], a.scale_log2, nmu))};
          lp[e & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lp[e & 1], false);
          w4[e] = __builtin_bit_cast(uint32_t, pp);
        }
        pb[kb][hh] = __builtin_bit_cast(bf16x8, u32x4{w4[0], w4[1], w4[2], w4[3]});
      }
    l += lp[0] + lp[1];
  };
  // O^T += V^T . P^T.  A operand for dim block db, k-step (kb, hh): the lane
  // needs V[key][32*db + lane%32] for the keys
  // 32*kb + 16*hh + 8*(e/4) + 4*half + e%4, e = 0..7: two transpose reads.
  auto pv = [&](int vof) {
    const int vb0 = vof + vbase[0], vb1 = vof + vbase[1];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const char* vb = smem + (32 * kb + 16 * hh) * kRowBytes;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + (vb0 ^ (db << 6))));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + (vb1 ^ (db << 6))));
          const bf16x8 va =
              __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb][hh], o[db], 0, 0, 0);
        }
  };
  // Step i with a next tile: S(i) in sc, S(i+1) into sn.
  auto step = [&](int i, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    top(i);
    scores(sn, k_tile(i + 1));
    probs(sc);
    // keep the probabilities ahead of the branch below, beside the score
    // products (the compiler would otherwise sink them into phase B)
    asm volatile("" ::"v"(pb[0][0]), "v"(pb[0][1]), "v"(pb[1][0]), "v"(pb[1][1]), "v"(l));
    if (needs_mask(i + 1)) mask(sn, key0_of(i + 1));
    pv(v_tile(i));
    if constexpr (kI8) dequant_ahead(i);
    raise_max(tile_max(sn));
  };
  // The last step: no next tile.
  auto last = [&](int i, f32x16 (&sc)[2]) {
    top(i);
    probs(sc);
    pv(v_tile(i));
  };

  // K(0) first (bf16: with K(1) and V(0) behind it; int8: the codes of
  // tiles 0 .. kStages - 1, of which 0 and 1 are dequantised here: K(0),
  // V(0), K(1)), then S(0).
  if constexpr (kI8) {
#pragma unroll
    for (int i = 0; i < kStages; ++i)
      if (i < nt) issue(i);
    wait_tiles<Lds::kVmPerTile>(max(0, min(kStages, nt) - 2));
    __syncthreads();                            // every wave's codes of tiles 0, 1 have landed
    dequant(0, 0, 0, key0_of(0));
    dequant(0, 0, 1, key0_of(0));
    if (nt > 1) dequant(1 % kStages, 1, 0, key0_of(1));
    __syncthreads();
  } else {
    issue(0, false);
    if (nt > 1) issue(1, false);
    issue(0, true);
    if (nt > 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * Lds::kVmPerTile));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(Lds::kVmPerTile));
    __syncthreads();                            // every wave's page of K(0) has landed
  }
  f32x16 sa[2], sb[2];
  scores(sa, k_tile(0));
  if (needs_mask(0)) mask(sa, key0_of(0));
  raise_max(tile_max(sa));
  int it = 0;
  for (; it + 2 < nt; it += 2) {              // two steps, the score registers swap roles
    step(it, sa, sb);
    step(it + 1, sb, sa);
  }
  if (it + 1 < nt) {
    step(it, sa, sb);
    last(it + 1, sb);
  } else {
    last(it, sa);
  }

  // Row sums: each half of the lanes summed its own keys.
  {
    const Halves h = halves32(l);
    l = h.lo + h.hi;
  }
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (bad) s_bad = 1;
  __syncthreads();
  const bool poisoned = bad_len || s_bad;
  const float nan = __builtin_nanf("");

  // O^T accumulator i of dim block db holds dim 32*db + 8*(i/4) + 4*half + i%4.
  uint32_t* orow = reinterpret_cast<uint32_t*>(
      a.out + ((int64_t)(q_lo + t_row) * a.Hq + g * G + j_row) * kD);
  if (a.splits == 1 || tk.ns == 1) {          // the group's keys lie in this one split
    if (!row_ok) return;
    const float inv = 1.f / l;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = 32 * db + 8 * i4 + 4 * half;
        uint32_t w0 = pack_bf16x2(o[db][4 * i4 + 0] * inv, o[db][4 * i4 + 1] * inv);
        uint32_t w1 = pack_bf16x2(o[db][4 * i4 + 2] * inv, o[db][4 * i4 + 3] * inv);
        if (poisoned) { w0 = 0x7fc07fc0u; w1 = 0x7fc07fc0u; }
        orow[d0 / 2] = w0;
        orow[d0 / 2 + 1] = w1;
      }
    return;
  }

  // Split path: write this split's unnormalised state for the workgroup's
  // rows with agent-coherent stores, wait for them, and count the arrival.
  // The last of the group's ns splits to arrive merges all of them, in split
  // order (the same arithmetic whichever split arrives last), and writes the
  // rows.  A partial is laid out [D/4][128 rows][4]: the four consecutive
  // dims a lane holds in each accumulator quad are 16 contiguous bytes, and
  // the 32 rows of a half-wave 512 contiguous bytes, so each lane writes and
  // reads its 64 values in 16 four-float accesses that coalesce.
  const int lrow = w * kRowsPerWave + (lane & 31);          // row within the tile
  const int64_t g0 = (int64_t)group * a.splits;              // the group's first split
  // dims 32 db + 8 k + 4 half + (0..3) of row lrow: quad 8 db + 2 k + half
  const uint32_t lane_quad = (uint32_t)((half * kRowsPerWG + lrow) * 4);   // floats
  {
    float* pacc = a.ws_acc + (g0 + ks) * kD * kRowsPerWG + lane_quad;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        f32x4 v = {o[db][4 * k], o[db][4 * k + 1], o[db][4 * k + 2], o[db][4 * k + 3]};
        if (poisoned) v = f32x4{nan, nan, nan, nan};
        ws_store4(pacc + (8 * db + 2 * k) * kRowsPerWG * 4, v);
      }
  }
  if (half == 0) ws_store2(a.ws_ml + 2 * ((g0 + ks) * kRowsPerWG + lrow), m, poisoned ? nan : l);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int* counter = a.counters + group;
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             tk.ns - 1;
  __syncthreads();
  if (!s_last) return;                        // uniform: not the last split
  // Leave the counter at zero for the next call on this workspace.
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!row_ok) return;
  // Online merge of the ns splits in split order, one split's loads (its
  // (m, l) and the lane's 64 dims of its partial, coherent loads waited for
  // together) at a time: two at a time measured no faster, and slower over
  // int8 pages.  The order is fixed, so the result does not depend on which
  // split came last.
  constexpr int kMB = 1;
  const int ns = tk.ns;
  float acc[4][16] = {};
  float Mr = kNegInf, Lr = 0.f;
  // The group's partials and (m, l) pairs as two buffer resources (the
  // buffer form takes the coherence bit as an operand the compiler tracks).
  const __amdgpu_buffer_rsrc_t acc_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      a.ws_acc + g0 * kD * kRowsPerWG, (short)0, ns * kD * kRowsPerWG * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t ml_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      a.ws_ml + 2 * g0 * kRowsPerWG, (short)0, ns * kRowsPerWG * 8, kBufferWord3);
  for (int s0 = 0; s0 < ns; s0 += kMB) {
    f32x2 mlv[kMB];
    f32x4 c[kMB][4][4];
#pragma unroll
    for (int j = 0; j < kMB; ++j) {
      const int sj = min(s0 + j, ns - 1);     // past the last split: loaded, not used
      mlv[j] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                             ml_rsrc, (sj * kRowsPerWG + lrow) * 8, 0, kCoherent));
      const int split_off = (sj * kD * kRowsPerWG + (int)lane_quad) * 4;   // bytes
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          c[j][db][k] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                         acc_rsrc, split_off + (8 * db + 2 * k) * kRowsPerWG * 16, 0, kCoherent));
    }
#pragma unroll
    for (int j = 0; j < kMB; ++j) {
      if (s0 + j >= ns) break;
      const float Mn = fmaxf(Mr, mlv[j][0]);
      const float Mu = (Mn == kNegInf) ? 0.f : Mn;
      const float r = fast_exp2(Mr - Mu), ws = fast_exp2(mlv[j][0] - Mu);
      Lr = __builtin_fmaf(mlv[j][1], ws, Lr * r);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[db][i] = __builtin_fmaf(c[j][db][i >> 2][i & 3], ws, acc[db][i] * r);
      Mr = Mn;
    }
  }
  const float inv = 1.f / Lr;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] *= inv;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = 32 * db + 8 * i4 + 4 * half;
      orow[d0 / 2] = pack_bf16x2(acc[db][4 * i4 + 0], acc[db][4 * i4 + 1]);
      orow[d0 / 2 + 1] = pack_bf16x2(acc[db][4 * i4 + 2], acc[db][4 * i4 + 3]);
    }
}

// Register budget: bf16 pages run two workgroups per CU (two waves per SIMD,
// so at most 256 registers each); int8 pages one (their code ring fills the
// LDS).
template <bool kI8>
__global__ void __launch_bounds__(kWaves * kWave, kI8 ? 1 : 2) prefill_kernel(const PrefillArgs a) {
  prefill_body<kI8>(a, blockIdx.x);
}

// Kernel arguments of a launch (host side).
inline PrefillArgs make_prefill_args(void* out, const void* q, const int32_t* cu_q,
                                     const void* k_cache, const void* v_cache,
                                     const float* k_scales, const float* v_scales,
                                     const int32_t* block_tables, const int32_t* ctx_lens, int B,
                                     int total_q, int max_q_len, int Hq, int Hkv, int num_blocks,
                                     int max_blocks, float scale, int window,
                                     const PrefillPlan& plan, void* workspace) {
  PrefillArgs a;
  a.out = static_cast<uint16_t*>(out);
  a.q = static_cast<const u32x4*>(q);
  a.cu_q = cu_q;
  a.k_cache = static_cast<const u32x4*>(k_cache);
  a.v_cache = static_cast<const u32x4*>(v_cache);
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.block_tables = block_tables;
  a.ctx_lens = ctx_lens;
  a.k_new = a.v_new = nullptr;
  char* ws = static_cast<char*>(workspace);
  const bool split = plan.splits > 1;
  a.ws_acc = split ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_ml = split ? reinterpret_cast<float*>(ws + plan.ws_acc_bytes) : nullptr;
  a.counters = split ? reinterpret_cast<int*>(ws + plan.ws_acc_bytes + plan.ws_ml_bytes) : nullptr;
  a.B = B; a.total_q = total_q; a.max_q_len = max_q_len;
  a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.num_blocks = num_blocks; a.max_blocks = max_blocks;
  a.qtiles = plan.qtiles;
  a.splits = plan.splits;
  a.tiles_per_split = plan.tiles_per_split;
  a.window = window;
  // The kernel needs a positive scale (it scales the row max, and masked
  // scores are -inf): a negative one flips q's sign instead, and 0 becomes
  // the least normal float, for which every product s * scale rounds to 0
  // or a subnormal as it does for 0, so every weight is exp2(0) = 1 alike.
  a.neg_q = scale < 0.f;
  a.scale_log2 = fabsf(scale) * 1.4426950408889634f;
  if (!(a.scale_log2 > 0.f)) a.scale_log2 = 1.17549435e-38f;
  return a;
}

}  // namespace
}  // namespace pf
}  // namespace pkv
