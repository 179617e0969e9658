// Slot mapping and KV append: integer and byte work, no floating point.
//
// Slot mapping follows the Module 12 page (qwen_serve/paged.py,
// PagedKVCache.write: position s lands in page blocks[s // 16] at offset
// s % 16; model.py forward: the step's tokens take positions start_pos ..
// start_pos+T-1).  Append is the same write as a row copy: pages are stored
// head-major ([page][KV head][16 slots][D]), so one token's K (or V) for all
// KV heads is Hkv rows of D*2 contiguous bytes, one per head, each copied
// with 16-byte moves.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

// One thread per appended token.  The owning sequence is found by binary
// search over cu_new_lens (B is small; the search is over at most B+1 ints).
__global__ void __launch_bounds__(256)
slot_mapping_kernel(int32_t* __restrict__ slots, const int32_t* __restrict__ block_tables,
                    const int32_t* __restrict__ cu_new, const int32_t* __restrict__ ctx_lens,
                    int B, int max_blocks, int total_new) {
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
  int page = p >> 4;
  int slot = -1;
  if (p >= 0 && page < max_blocks) {
    int blk = block_tables[(int64_t)b * max_blocks + page];
    if (blk >= 0) slot = blk * kPage + (p & (kPage - 1));
  }
  slots[t] = slot;
}

// Work item = one 16-byte chunk of one token's K or V row of one KV head.
// Consecutive threads take consecutive chunks of a token's [Hkv][D] row in
// k_new, so the read is fully coalesced and each head's 256-byte row lands
// as a contiguous run in its page.
__global__ void __launch_bounds__(256)
append_kernel(const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
              const int32_t* __restrict__ slots, u32x4* __restrict__ k_cache,
              u32x4* __restrict__ v_cache, int64_t n_items, int Hkv, int chunks_per_head,
              int64_t num_slots) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int chunks_per_row = Hkv * chunks_per_head;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_items; i += stride) {
    const int64_t t = i / (2 * chunks_per_row);
    const int row_item = (int)(i % (2 * chunks_per_row));
    const int which = row_item / chunks_per_row;
    const int r = row_item % chunks_per_row;     // chunk within the token's [Hkv][D] row
    const int h = r / chunks_per_head;
    const int c = r % chunks_per_head;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot / kPage, off = slot % kPage;
    const u32x4* src = which ? v_new : k_new;
    u32x4* dst = which ? v_cache : k_cache;
    dst[((blk * Hkv + h) * kPage + off) * chunks_per_head + c] = src[t * chunks_per_row + r];
  }
}

hipError_t launch_slot_mapping(int32_t* slots, const int32_t* block_tables, const int32_t* cu_new,
                               const int32_t* ctx_lens, int B, int max_blocks, int total_new,
                               hipStream_t stream) {
  if (total_new == 0) return hipSuccess;
  dim3 grid((total_new + 255) / 256);
  hipLaunchKernelGGL(slot_mapping_kernel, grid, dim3(256), 0, stream, slots, block_tables, cu_new,
                     ctx_lens, B, max_blocks, total_new);
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
