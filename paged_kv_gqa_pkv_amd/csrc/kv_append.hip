// Slot mapping and KV append: integer and byte work, no floating point.
//
// Slot mapping follows the Module 12 page (qwen_serve/paged.py,
// PagedKVCache.write: position s lands in page blocks[s // 16] at offset
// s % 16; model.py forward: the step's tokens take positions start_pos ..
// start_pos+T-1).  Append is the same write as a row copy: pages are stored
// token-major as in paged.py ([page][16 slots][KV head][D]), so one token's K
// (or V) for all KV heads is one contiguous run of Hkv*D*2 bytes in its page,
// copied with 16-byte moves.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

// One thread per appended token.  The owning sequence is found by binary
// search over cu_new_lens (B is small; the search is over at most B+1 ints).
__global__ void __launch_bounds__(256)
slot_mapping_kernel(int32_t* __restrict__ slots, const int32_t* __restrict__ block_tables,
                    const int32_t* __restrict__ cu_new, const int32_t* __restrict__ ctx_lens,
                    int B, int max_blocks, int total_new, int window) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total_new) return;
  int lo = 0, hi = B;               // find b with cu[b] <= t < cu[b+1]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu_new[mid] <= t) lo = mid; else hi = mid;
  }
  int b = lo;
  int n_new = cu_new[b + 1] - cu_new[b];
  int p = ctx_lens[b] - n_new + (t - cu_new[b]);
  // A ring of `window` tokens (Module 04 page, section 4) writes position p at
  // ring index p % window.
  if (window > 0 && p >= 0) p %= window;
  int page = p >> 4;
  int slot = -1;
  if (p >= 0 && page < max_blocks) {
    int blk = block_tables[(int64_t)b * max_blocks + page];
    // Slots are int32: an id at or above kMaxSlotBlocks has no slot and is
    // treated like a missing page.
    if (blk >= 0 && blk < kMaxSlotBlocks) slot = blk * kPage + (p & (kPage - 1));
  }
  slots[t] = slot;
}

// Grid-stride row copy (append_rows): consecutive threads take consecutive
// 16-byte chunks of a token's K or V row.
__global__ void __launch_bounds__(256)
append_kernel(const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
              const int32_t* __restrict__ slots, u32x4* __restrict__ k_cache,
              u32x4* __restrict__ v_cache, int64_t n_items, int Hkv, int chunks_per_head,
              int64_t num_slots) {
  append_rows(k_new, v_new, slots, k_cache, v_cache, n_items, Hkv, chunks_per_head, num_slots,
              (int64_t)blockIdx.x * blockDim.x + threadIdx.x, (int64_t)gridDim.x * blockDim.x);
}

// int8 append: quantise each new (token, KV head) row as the Module 04 page
// does (kv_cache.py listing, section 5, KV8Cache.write), in float32:
//   scale = max_d |x_d| / 127 + 1e-8,   code_d = clip(rint(x_d / scale), -127, 127)
// with round half to even, so the codes and scale match the page's numpy
// float32 arithmetic bit for bit.  16 lanes own one row of 128 values (8 per
// lane): the row max is a DPP reduction inside the 16-lane row, each lane
// writes its 8 codes (8 bytes), and the first lane writes the scale.  Codes
// are token-major like the bf16 pools ([page][16 slots][KV head][D]); the
// scales (the listing's ks and vs [L, cap, H_kv], one layer, cap cut into
// pages) sit at [page][KV head][slot] of k_scales or v_scales, so the 16
// scales a KV head needs from a page are one 64-byte run.  The arithmetic
// is int8_row_scale / int8_code (correctly rounded quotients without a
// division per value).
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, dpp_f<kDppQuadSwap1>(x));
  x = fmaxf(x, dpp_f<kDppQuadSwap2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  return fmaxf(x, dpp_f<kDppRowRor8>(x));
}

__global__ void __launch_bounds__(256)
append_int8_kernel(const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
                   const int32_t* __restrict__ slots, uint2* __restrict__ k_codes,
                   uint2* __restrict__ v_codes, float* __restrict__ k_scales,
                   float* __restrict__ v_scales, int64_t n_rows, int Hkv, int64_t num_slots) {
  const int sub = threadIdx.x & 15;                    // lane within the row group
  // r = (t * 2 + which) * Hkv + h, one row per 16-lane group: all 16 lanes
  // share r, so the DPP reduction below only reads lanes of the same row.
  const int64_t r = (int64_t)blockIdx.x * (blockDim.x / 16) + (threadIdx.x >> 4);
  if (r >= n_rows) return;
  const int h = (int)(r % Hkv);
  const int which = (int)((r / Hkv) & 1);
  const int64_t t = r / (2 * (int64_t)Hkv);
  const int64_t slot = slots[t];
  const u32x4 w = (which ? v_new : k_new)[(t * Hkv + h) * 16 + sub];
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) { x[2 * i] = bf16lo(w[i]); x[2 * i + 1] = bf16hi(w[i]); }
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(x[i]));
  mx = max16(mx);
  const float scale = int8_row_scale(mx);
  const float y = 1.0f / scale;
  uint32_t pk[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) pk[i >> 2] |= int8_code(x[i], scale, y) << (8 * (i & 3));
  if (slot < 0 || slot >= num_slots) return;
  const int64_t row = slot * Hkv + h;                             // codes row (128 B)
  (which ? v_codes : k_codes)[row * 16 + sub] = make_uint2(pk[0], pk[1]);
  const int64_t srow = ((slot / kPage) * Hkv + h) * kPage + slot % kPage;
  if (sub == 0) (which ? v_scales : k_scales)[srow] = scale;
}

hipError_t launch_append_int8(const void* k_new, const void* v_new, const int32_t* slots,
                              void* k_codes, void* v_codes, float* k_scales, float* v_scales,
                              int T, int num_blocks, int Hkv, int D, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (D != 128) return hipErrorInvalidValue;       // 16 lanes x 8 values per row
  const int64_t n_rows = (int64_t)T * 2 * Hkv;
  const int64_t blocks = (n_rows + 15) / 16;          // one row per 16 lanes
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(append_int8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const u32x4*)k_new, (const u32x4*)v_new, slots, (uint2*)k_codes,
                     (uint2*)v_codes, k_scales, v_scales, n_rows, Hkv,
                     (int64_t)num_blocks * kPage);
  return hipGetLastError();
}

// Copy-on-write / fork page copy (Module 12 page, paged.py:
// SequenceCache._cow_copy and fork_from copy block src to a fresh block dst
// in every layer, K and V).  One work item is one 16-byte chunk of one block
// of one layer of one pool; consecutive threads take consecutive chunks, so
// reads and writes are contiguous runs of the block.  Pairs whose ids fall
// outside the pool are skipped.
__global__ void __launch_bounds__(256)
copy_blocks_kernel(char* __restrict__ k_pool, char* __restrict__ v_pool,
                   const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
                   int64_t n_items, int64_t chunks_per_block, int pools, int n_layers,
                   int64_t layer_stride, int num_blocks) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t block_bytes = chunks_per_block * 16;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_items; i += stride) {
    const int64_t c = i % chunks_per_block;
    int64_t rest = i / chunks_per_block;
    const int pool = (int)(rest % pools);
    rest /= pools;
    const int layer = (int)(rest % n_layers);
    const int64_t pair = rest / n_layers;
    const int s = src[pair], d = dst[pair];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) continue;
    char* base = (pool ? v_pool : k_pool) + layer * layer_stride;
    reinterpret_cast<u32x4*>(base + d * block_bytes)[c] =
        reinterpret_cast<const u32x4*>(base + s * block_bytes)[c];
  }
}

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst,
                              int n_pairs, int num_blocks, int64_t block_bytes, int n_layers,
                              int64_t layer_stride, hipStream_t stream) {
  if (n_pairs == 0 || n_layers == 0 || block_bytes == 0) return hipSuccess;
  const int pools = v_pool ? 2 : 1;
  const int64_t cpb = block_bytes / 16;
  const int64_t n_items = (int64_t)n_pairs * n_layers * pools * cpb;
  int64_t blocks = (n_items + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<char*>(k_pool), static_cast<char*>(v_pool), src, dst, n_items,
                     cpb, pools, n_layers, layer_stride, num_blocks);
  return hipGetLastError();
}

hipError_t launch_slot_mapping(int32_t* slots, const int32_t* block_tables, const int32_t* cu_new,
                               const int32_t* ctx_lens, int B, int max_blocks, int total_new,
                               int window, hipStream_t stream) {
  if (total_new == 0) return hipSuccess;
  dim3 grid((total_new + 255) / 256);
  hipLaunchKernelGGL(slot_mapping_kernel, grid, dim3(256), 0, stream, slots, block_tables, cu_new,
                     ctx_lens, B, max_blocks, total_new, window);
  return hipGetLastError();
}

hipError_t launch_append(const void* k_new, const void* v_new, const int32_t* slots,
                         void* k_cache, void* v_cache, int T, int num_blocks, int Hkv, int D,
                         hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int chunks_per_head = D * 2 / 16;
  const int64_t n_items = (int64_t)T * 2 * Hkv * chunks_per_head;
  int64_t blocks = (n_items + 255) / 256;
  if (blocks > 8192) blocks = 8192;  // grid-stride beyond 32 waves per CU
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const u32x4*)k_new, (const u32x4*)v_new, slots, (u32x4*)k_cache,
                     (u32x4*)v_cache, n_items, Hkv, chunks_per_head, (int64_t)num_blocks * kPage);
  return hipGetLastError();
}

}  // namespace pkv
