// Host-side launchers of the gfx950 kernels (internal; the C ABI sits above).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// window > 0: each sequence's pages form a ring of `window` tokens.
hipError_t launch_slot_mapping(int32_t* slots, const int32_t* block_tables, const int32_t* cu_new,
                               const int32_t* ctx_lens, int B, int max_blocks, int total_new,
                               int window, hipStream_t stream);

hipError_t launch_append(const void* k_new, const void* v_new, const int32_t* slots,
                         void* k_cache, void* v_cache, int T, int num_blocks, int Hkv, int D,
                         hipStream_t stream);

// Block copy for copy-on-write and fork: for each pair, block dst of every
// layer of k_pool (and v_pool if not null) becomes a copy of block src.
// Pool l starts at pool + l * layer_stride; blocks are block_bytes apart.
hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst,
                              int n_pairs, int num_blocks, int64_t block_bytes, int n_layers,
                              int64_t layer_stride, hipStream_t stream);

// q/k RMSNorm + RoPE + append of the rotated k and of v into their slots
// (slots found from the tables, as launch_slot_mapping does; written to
// `slots` when it is not null).
hipError_t launch_qk_norm_rope_append(void* q_out, const void* q_in, const void* k_in,
                                      const void* v_in, const void* q_norm_w,
                                      const void* k_norm_w, const void* cos_table,
                                      const void* sin_table, int max_pos,
                                      const int32_t* block_tables, const int32_t* cu_new,
                                      const int32_t* ctx_lens, int32_t* slots, void* k_cache,
                                      void* v_cache, int B, int max_blocks, int T,
                                      int num_blocks, int Hq, int Hkv, float eps,
                                      hipStream_t stream);

// Split plan of a decode call: S splits of pages_per_split pages each, one
// workgroup per (sequence, split, group of heads_per_wg KV heads) with
// `parts` waves per head, each over pages_per_split / parts pages.
struct DecodePlan {
  int splits;
  int pages_per_split;
  int heads_per_wg;
  int parts;
  size_t ws_ml_bytes;    // float2 (m, l) [B][Hq][S]
  size_t ws_acc_bytes;   // float [B][Hq][S][D]
  size_t ws_counter_bytes;  // int [B][Hkv / heads_per_wg] split arrival counters
  size_t ws_bytes;       // total, 0 for a single pass
};

DecodePlan plan_decode(int B, int Hq, int Hkv, int max_context_len, int num_cus);

hipError_t launch_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* ctx_lens, int B, int Hq,
                         int Hkv, int num_blocks, int max_blocks, float scale, int window,
                         const DecodePlan& plan, void* workspace, hipStream_t stream);

// Decode with the step's append fused in: position context_lens[b] - 1 of
// each sequence takes its K/V rows from k_new / v_new [B][Hkv][D] (not from
// the pool), and the call writes them into that position's slot.  Same plan
// and workspace as launch_decode.
hipError_t launch_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, const int32_t* block_tables,
                                const int32_t* ctx_lens, int B, int Hq, int Hkv, int num_blocks,
                                int max_blocks, float scale, const DecodePlan& plan,
                                void* workspace, hipStream_t stream);

// The same over int8 pages: the new rows are quantised as launch_append_int8
// quantises them and written with their scales.
hipError_t launch_decode_append_int8(void* out, const void* q, const void* k_new,
                                     const void* v_new, void* k_codes, void* v_codes,
                                     float* k_scales, float* v_scales,
                                     const int32_t* block_tables, const int32_t* ctx_lens, int B,
                                     int Hq, int Hkv, int num_blocks, int max_blocks, float scale,
                                     const DecodePlan& plan, void* workspace,
                                     hipStream_t stream);

// Decode with the split buffers in the library's own per-device array
// (no caller workspace).  noalloc_fits tells whether a plan fits that array.
bool noalloc_fits(const DecodePlan& plan, int B, int Hkv);
hipError_t launch_decode_noalloc(void* out, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* ctx_lens, int B, int Hq, int Hkv, int num_blocks,
                                 int max_blocks, float scale, const DecodePlan& plan,
                                 hipStream_t stream);

// Decode over int8 pages (codes in the bf16 page order; float32 scales
// [num_blocks][Hkv][16] for K and for V); same plan and workspace as
// launch_decode.
hipError_t launch_decode_int8(void* out, const void* q, const void* k_codes, const void* v_codes,
                              const float* k_scales, const float* v_scales,
                              const int32_t* block_tables,
                              const int32_t* ctx_lens, int B, int Hq, int Hkv, int num_blocks,
                              int max_blocks, float scale, const DecodePlan& plan,
                              void* workspace, hipStream_t stream);

hipError_t launch_append_int8(const void* k_new, const void* v_new, const int32_t* slots,
                              void* k_codes, void* v_codes, float* k_scales, float* v_scales,
                              int T, int num_blocks, int Hkv, int D, hipStream_t stream);

// Key-split plan of a prefill call: row tiles of 128 (token, head) rows,
// key ranges of tiles_per_split 64-key tiles.
struct PrefillPlan {
  bool ok;                  // false: the context is longer than the kernel supports
  int qtiles;
  int splits;
  int tiles_per_split;
  size_t ws_acc_bytes;      // float [groups][S][D/4][128][4]
  size_t ws_ml_bytes;       // float [groups][S][128][2]
  size_t ws_counter_bytes;  // int [groups], split arrivals (zero between calls)
  size_t ws_bytes;          // total, 0 without splits
};

PrefillPlan plan_prefill(int B, int max_q_len, int Hq, int Hkv, int max_context_len, int num_cus);

// k_scales null: bf16 pages; else int8 codes in k_cache / v_cache with
// their scales in k_scales / v_scales.
hipError_t launch_prefill(void* out, const void* q, const int32_t* cu_q, const void* k_cache,
                          const void* v_cache, const float* k_scales, const float* v_scales,
                          const int32_t* block_tables,
                          const int32_t* ctx_lens, int B, int total_q, int max_q_len, int Hq,
                          int Hkv, int num_blocks, int max_blocks, float scale, int window,
                          const PrefillPlan& plan, void* workspace, hipStream_t stream);

// Mixed step (bf16 pages): the chunk of launch_prefill and the decode of
// launch_decode in one grid, each with its own plan and workspace.  Needs a
// decode plan of 4 page-part waves and a group size G = Hq / Hkv of at most
// 4 (mixed_plan_fits).
bool mixed_plan_fits(const DecodePlan& dplan, int G);
hipError_t launch_prefill_decode(void* out_p, const void* q_p, const int32_t* cu_q,
                                 const int32_t* bt_p, const int32_t* ctx_p, int B_p, int total_q,
                                 int max_q_len, const PrefillPlan& pplan, void* ws_p,
                                 void* out_d, const void* q_d, const int32_t* bt_d,
                                 const int32_t* ctx_d, int B_d, const DecodePlan& dplan,
                                 void* ws_d, const void* k_cache, const void* v_cache, int Hq,
                                 int Hkv, int num_blocks, int max_blocks, float scale,
                                 hipStream_t stream);
// The same over int8 pages (codes and head-major scales as for
// launch_prefill / launch_decode_int8), one workgroup per CU.
hipError_t launch_prefill_decode_int8(void* out_p, const void* q_p, const int32_t* cu_q,
                                      const int32_t* bt_p, const int32_t* ctx_p, int B_p,
                                      int total_q, int max_q_len, const PrefillPlan& pplan,
                                      void* ws_p, void* out_d, const void* q_d,
                                      const int32_t* bt_d, const int32_t* ctx_d, int B_d,
                                      const DecodePlan& dplan, void* ws_d, const void* k_codes,
                                      const void* v_codes, const float* k_scales,
                                      const float* v_scales, int Hq, int Hkv, int num_blocks,
                                      int max_blocks, float scale, hipStream_t stream);
// The same with the step's append in the grid: the chunk reads its own rows
// from k_new ([total_q + B_d][Hkv][D]: the chunk rows in cu_q order, then one
// row per decode sequence), the decode half takes its rows from there and
// writes them into their slots, and the chunk rows are copied into
// slot_mapping[0 .. total_q).  Same plans and workspaces.
hipError_t launch_prefill_decode_append(
    void* out_p, const void* q_p, const int32_t* cu_q, const int32_t* bt_p, const int32_t* ctx_p,
    int B_p, int total_q, int max_q_len, const PrefillPlan& pplan, void* ws_p, void* out_d,
    const void* q_d, const int32_t* bt_d, const int32_t* ctx_d, int B_d, const DecodePlan& dplan,
    void* ws_d, const void* k_new, const void* v_new, const int32_t* slot_mapping,
    void* k_cache, void* v_cache, int Hq, int Hkv, int num_blocks, int max_blocks, float scale,
    hipStream_t stream);

}  // namespace pkv
