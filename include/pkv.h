/*
 * pkv.h -- paged grouped-query attention for MI355X (gfx950): C ABI.
 *
 * Pages cited below:
 *   [P1] "Module 12: Final project - mini inference engine" (LLM Inference
 *        Systems course), listings qwen_serve/paged.py and qwen_serve/model.py.
 *   [P2] "Module 04: KV cache and memory arithmetic" (same course).
 *   [P3] "Inference Optimization" (AI Engineering from Scratch), section
 *        "Paged Attention".
 *
 * Data layout (all tensors contiguous, row-major, bf16 unless stated):
 *   k_cache, v_cache   [num_blocks][block_size=16][Hkv][D]   one layer's page
 *                      pool, the per-layer slice of [P1] paged.py's
 *                      [n_layers, capacity, block_size, n_kv_heads,
 *                      head_dim]: the row of (page b, slot s, KV head g)
 *                      starts at ((b*16 + s)*Hkv + g)*D elements, so one
 *                      token's K (or V) for all KV heads is Hkv*D contiguous
 *                      values and flat slot b*16 + s is row block
 *                      b*16 + s of [num_blocks*16][Hkv][D].
 *   block_tables       int32 [B][max_blocks_per_seq]: logical page i of
 *                      sequence b lives in physical page block_tables[b][i]
 *                      ([P1] SequenceCache.blocks; [P3] page table).  Entries
 *                      past a sequence's last page are never read.  Positions
 *                      are int32, so max_blocks_per_seq < 2^27 (else
 *                      PKV_EINVAL).
 *   context_lens       int32 [B]: tokens in each sequence's pages, counting
 *                      the tokens appended in this step (append runs first).
 *
 * Ownership: every pointer is a device pointer owned by the caller (except
 * where "host" is stated).  The library allocates nothing, keeps no pointer
 * after a call returns and enqueues all work on `stream` (a hipStream_t;
 * NULL is the default stream): buffers must stay alive until the stream has
 * passed the work.  Calls on one stream are ordered; calls on different
 * streams that touch the same memory need the caller's synchronisation.
 *
 * Errors: every entry point returns PKV_OK (0) or a negative code and never
 * throws.  Argument and shape errors are detected on the host before any
 * launch (nothing is enqueued).  The contents of index arrays live on the
 * device and are not inspected on the hot path: kernels stay inside their
 * buffers whatever the indices hold (an out-of-range block id or length
 * makes the affected outputs NaN; an out-of-range slot is skipped).  With
 * the environment variable PKV_VALIDATE=1 each call first copies its index
 * arrays to the host (synchronising `stream`) and rejects bad contents with
 * PKV_EVALIDATE.  pkv_last_error() returns a thread-local message for the
 * last non-OK return on the calling thread.
 *
 * Supported geometry: block_size 16 ([P1] default --block-size 16), D = 128
 * (every model the pages name), Hq % Hkv == 0 with Hq/Hkv in {1,2,4,8};
 * anything else returns PKV_EUNSUPPORTED.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,        /* null pointer, negative size, inconsistent shapes */
  PKV_EUNSUPPORTED = -2,  /* geometry outside the supported set */
  PKV_EWORKSPACE = -3,    /* decode workspace smaller than required */
  PKV_ELAUNCH = -4,       /* the HIP runtime reported an error */
  PKV_EVALIDATE = -5      /* PKV_VALIDATE=1 found bad index contents */
};

#define PKV_BLOCK_SIZE 16
#define PKV_HEAD_DIM 128

/*
 * Slot mapping ([P1] paged.py PagedKVCache.write: position s goes to
 * (blocks[s // block_size], s % block_size); model.py forward: a step's
 * tokens take positions start_pos .. start_pos+T-1, start_pos being the
 * committed length).
 *
 * Sequence b appends n_b = cu_new_lens[b+1] - cu_new_lens[b] tokens which end
 * its context, so token j (0 <= j < n_b) sits at p = context_lens[b] - n_b + j
 * and gets the flat physical slot
 *     slot_mapping[cu_new_lens[b] + j] = block_tables[b][p / 16] * 16 + p % 16.
 * A position that would fall outside the table (p < 0 or p / 16 >=
 * max_blocks_per_seq), or whose table entry is negative or at least 2^27
 * (its slot would not fit in int32), yields -1 (skip).
 *   slot_mapping  int32 [total_new] (output)
 *   cu_new_lens   int32 [B+1], nondecreasing, cu_new_lens[0] = 0,
 *                 cu_new_lens[B] = total_new
 */
int pkv_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables,
                     const int32_t* cu_new_lens, const int32_t* context_lens,
                     int32_t B, int32_t max_blocks_per_seq, int32_t total_new,
                     int32_t block_size, void* stream);

/*
 * KV append ([P1] paged.py PagedKVCache.write; model.py forward writes the
 * step's K/V into the pages).  A bit-exact scatter of rows:
 *     k_cache[slot / 16][slot % 16][:][:] = k_new[t][:][:]   (all KV heads; same for V)
 * for every t with 0 <= slot = slot_mapping[t] < num_blocks*16; other slots
 * (negative = padding) are skipped.  Slots must be distinct (duplicates race;
 * PKV_VALIDATE=1 rejects them).
 *   k_new, v_new  bf16 [T][Hkv][D]
 */
int pkv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping,
               void* k_cache, void* v_cache, int32_t T, int32_t num_blocks,
               int32_t Hkv, int32_t D, int32_t block_size, void* stream);

/*
 * Block copy for copy-on-write and fork ([P1] paged.py: SequenceCache._cow_copy
 * and fork_from copy block src to a fresh block nb in every layer,
 * k[:, nb] = k[:, src] and the same for v; [P3] "Paged Attention": a shared
 * page is copied before it is written).  For every pair i, block
 * dst_blocks[i] of every layer of k_pool (and of v_pool unless it is NULL)
 * becomes a bit copy of block src_blocks[i].
 *   k_pool, v_pool   device memory holding n_layers pools, layer l starting
 *                    at pool + l * layer_stride_bytes, block b of a layer at
 *                    b * block_bytes from its start (any page format: bf16
 *                    pools have block_bytes = 16*Hkv*D*2, int8 codes
 *                    16*Hkv*D, int8 scale arrays 16*Hkv*4)
 *   src_blocks, dst_blocks  int32 [n_pairs], device
 * Pointers, block_bytes and layer_stride_bytes must be multiples of 16.
 * Destinations must be distinct and no destination may be a source (the
 * pairs run in parallel; PKV_VALIDATE=1 rejects such pairs and ids outside
 * [0, num_blocks)); without it, pairs with an id outside the pool are skipped.
 */
int pkv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src_blocks,
                    const int32_t* dst_blocks, int32_t n_pairs, int32_t num_blocks,
                    int64_t block_bytes, int32_t n_layers, int64_t layer_stride_bytes,
                    void* stream);

/*
 * Workspace for pkv_attn_decode: bytes of device memory the split-context
 * path needs for the given shape (0 when the call runs in a single pass).
 * Depends on the current device's compute-unit count.  Returns 0 for
 * unsupported shapes as well; pkv_attn_decode reports those.
 */
size_t pkv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t max_context_len);

/* Number of context splits pkv_attn_decode uses for this shape (>= 1). */
int32_t pkv_decode_num_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                              int32_t max_context_len);

/*
 * Decode attention ([P2] section 1: o_n = softmax(q_n K_{0:n}^T / sqrt(d_head))
 * V_{0:n}; [P1] model.py forward with T = 1; GQA: query head h reads KV head
 * h / (Hq/Hkv), [P1] q.view(T, n_kv, group, D)).
 *     out[b][h][:] = sum_p w_p V_b[p][h/G][:],  w = softmax_p(scale * <q[b][h], K_b[p][h/G]>)
 * over positions p < context_lens[b] read through block_tables[b].
 * context_lens[b] == 0 gives zeros; a length past the table or beyond what
 * max_context_len planned for gives NaN.  fp32 accumulation, bf16 output.
 * One kernel launch: long contexts are cut into splits whose partial
 * softmax states are merged, in split order, by the last split to finish.
 *   out, q        bf16 [B][Hq][D]; must not overlap
 *   scale         normally 1/sqrt(D)
 *   max_context_len  host-side upper bound of context_lens (plans the splits)
 *   workspace     device buffer of at least pkv_decode_workspace_bytes(...)
 *                 bytes (may be NULL when that is 0).  It must be
 *                 zero-filled before its first use; every call leaves it
 *                 ready for the next (its arrival counters back at zero).
 *                 Calls that may overlap in time need separate workspaces.
 */
int pkv_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                    int32_t num_blocks, int32_t max_blocks_per_seq,
                    int32_t max_context_len, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode with the step's append fused in ([P1] model.py forward: each layer
 * reads the cached prefix, concatenates the step's own k/v to it, attends,
 * and writes the step's k/v into the cache).  Every sequence b appends one
 * token, at position p = context_lens[b] - 1 (context_lens count it, as for
 * pkv_attn_decode): the call is pkv_append of k_new[b] / v_new[b] into the
 * slot of p, found from block_tables as pkv_slot_mapping finds it (no row is
 * written where that gives -1), followed by pkv_attn_decode, with the same
 * outputs, except that position p's K/V rows are taken from k_new / v_new
 * instead of being read back from the pool (the same bits).  One launch; no
 * slot mapping needed.  Same errors, split plan and workspace as
 * pkv_attn_decode (pkv_decode_workspace_bytes applies unchanged).
 *   k_new, v_new     bf16 [B][Hkv][D], the step's rows
 *   k_cache, v_cache the pools, read and written ([num_blocks][16][Hkv][D])
 */
int pkv_attn_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                           void* k_cache, void* v_cache, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t block_size, int32_t num_blocks,
                           int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Size of the per-GPU array of pkv_attn_decode_noalloc and of its counter
 * region (16 MiB, 64 KiB). */
#define PKV_NOALLOC_SCRATCH_BYTES (16u << 20)
#define PKV_NOALLOC_COUNTER_BYTES (64u << 10)

/*
 * Decode attention for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that forbid allocation, harnesses
 * that forbid hipMalloc).  Same arguments, outputs and error behaviour as
 * pkv_attn_decode minus the workspace: the split path keeps its partials
 * and arrival counters in one array the library holds on each GPU (its
 * first call on a device resolves that array and clears its counters with a
 * small kernel on `stream`; the array lives until the process ends).  The
 * call allocates nothing.  Shapes whose split plan needs more than
 * PKV_NOALLOC_SCRATCH_BYTES - PKV_NOALLOC_COUNTER_BYTES bytes of partials,
 * or more than PKV_NOALLOC_COUNTER_BYTES / 4 (sequence, KV head) pairs,
 * return PKV_EWORKSPACE before anything is enqueued (pkv_attn_decode with a
 * workspace covers them).  All calls on one GPU share the array: calls that
 * may overlap in time on one GPU (other streams, other threads) race and
 * must be serialised by the caller.
 */
int pkv_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                            int32_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t max_context_len, float scale, void* stream);

/*
 * Workspace for pkv_attn_prefill_chunk: bytes of device memory the call needs
 * for this shape (0 when it runs without key splits).  Depends on the current
 * device's compute-unit count.  0 for unsupported shapes as well.
 */
size_t pkv_prefill_workspace_bytes(int32_t B, int32_t max_q_len, int32_t Hq, int32_t Hkv,
                                   int32_t D, int32_t max_context_len);

/*
 * Causal chunked-prefill attention ([P1] model.py forward with T > 1: mask
 * kpos <= qpos on absolute positions; [P1] "Why chunked prefill": prompt
 * chunks of up to 512 tokens).  Sequence b owns query rows
 * cu_q_lens[b] .. cu_q_lens[b+1]-1; they are the last T_b positions of its
 * context, so row t sits at position context_lens[b] - T_b + t and attends to
 * keys 0 .. that position, read through block_tables[b] (the chunk's own K/V
 * must already be appended).  T_b > context_lens[b] makes that sequence's
 * rows NaN; a sequence whose rows fall outside [0, total_q) or number more
 * than max_q_len is skipped (its rows are left untouched).  bf16 MFMA with
 * fp32 accumulation and fp32 softmax statistics, bf16 output.  Contexts up
 * to 131072 tokens (longer: PKV_EUNSUPPORTED).
 *   out, q        bf16 [total_q][Hq][D]; must not overlap
 *   cu_q_lens     int32 [B+1], nondecreasing, cu_q_lens[0] = 0,
 *                 cu_q_lens[B] = total_q
 *   max_q_len     host-side upper bound of T_b
 *   max_context_len  host-side upper bound of context_lens (plans key splits)
 *   workspace     device buffer of at least pkv_prefill_workspace_bytes(...)
 *                 bytes (may be NULL when that is 0): the key splits'
 *                 partial results and one arrival counter per (row tile,
 *                 KV head).  One launch: the last split of a row tile to
 *                 finish merges the partials in split order.  The buffer
 *                 must be zero-filled before its first use; every call
 *                 leaves its counters back at zero for the next.  Calls
 *                 that may overlap in time need separate workspaces.
 */
int pkv_attn_prefill_chunk(void* out, const void* q, const int32_t* cu_q_lens,
                           const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int32_t B, int32_t total_q, int32_t max_q_len,
                           int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                           int32_t num_blocks, int32_t max_blocks_per_seq,
                           int32_t max_context_len, float scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * The attention of a mixed step ([P1] "Why chunked prefill": one scheduler
 * step carries a decode token for each decoding sequence beside prompt
 * chunks; [P1] model.py forward runs attention for all of them over the
 * pages) in one call: pkv_attn_prefill_chunk over the prefill sequences and
 * pkv_attn_decode over the decode sequences, on the same pools, with the
 * same outputs bit for bit.  Group sizes Hq/Hkv of 1, 2 and 4 run as one
 * launch whose grid holds both kinds of workgroup (the two halves overlap on
 * the chip instead of running one after the other); group size 8, or a call
 * with one half empty, runs the two launches in order.
 *   out_prefill, q_prefill, cu_q_lens, block_tables_prefill,
 *   context_lens_prefill, B_prefill, total_q, max_q_len,
 *   max_context_len_prefill     as out, q, cu_q_lens, block_tables,
 *                               context_lens, B, total_q, max_q_len and
 *                               max_context_len of pkv_attn_prefill_chunk
 *   out_decode, q_decode, block_tables_decode, context_lens_decode,
 *   B_decode, max_context_len_decode   as those of pkv_attn_decode
 *   k_cache, v_cache, Hq, Hkv, D, block_size, num_blocks, scale
 *                               shared by both halves
 *   max_blocks_per_seq          row width of both block tables
 *   prefill_workspace           pkv_prefill_workspace_bytes(B_prefill,
 *                               max_q_len, ...) bytes, as for the chunk call
 *   decode_workspace            pkv_decode_workspace_bytes(B_decode, ...)
 *                               bytes, as for the decode call; both
 *                               zero-filled before their first use and left
 *                               so, and distinct
 * Errors: those of either call (checked before anything is enqueued), and
 * PKV_EINVAL if the two outputs or the two (non-empty) workspaces coincide.
 * The step's K/V rows must be appended before the call.
 */
int pkv_attn_prefill_decode(void* out_prefill, const void* q_prefill, const int32_t* cu_q_lens,
                            const int32_t* block_tables_prefill,
                            const int32_t* context_lens_prefill, int32_t B_prefill,
                            int32_t total_q, int32_t max_q_len, int32_t max_context_len_prefill,
                            void* out_decode, const void* q_decode,
                            const int32_t* block_tables_decode,
                            const int32_t* context_lens_decode, int32_t B_decode,
                            int32_t max_context_len_decode, const void* k_cache,
                            const void* v_cache, int32_t Hq, int32_t Hkv, int32_t D,
                            int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                            float scale, void* prefill_workspace, size_t prefill_workspace_bytes,
                            void* decode_workspace, size_t decode_workspace_bytes,
                            void* stream);

/*
 * A mixed step's append and attention in one call ([P1] model.py forward:
 * each layer writes the step's K/V into the cache and attends over the
 * cached prefix plus those rows): pkv_append of the step's rows followed by
 * pkv_attn_prefill_decode, in one launch for group sizes 1, 2 and 4.  The
 * chunk workgroups read their chunk's own rows from k_new / v_new instead of
 * the pool (the same bits, so the prefill output is that of the two calls
 * bit for bit); the decode workgroups take their sequence's new row from
 * k_new / v_new and write it into its slot, found from the block table as
 * pkv_attn_decode_append finds it (decode outputs equal those of the two
 * calls up to the order of float32 sums); further workgroups in the same
 * grid copy the chunk rows into their slots.  Nothing in the grid reads a
 * slot the grid writes.  Group size 8, or one half empty, runs pkv_append,
 * then the attention launches in order.
 *   k_new, v_new   bf16 [total_q + B_decode][Hkv][D]: the chunk rows of the
 *                  prefill sequences in cu_q_lens order, then one row per
 *                  decode sequence
 *   slot_mapping   int32 [total_q + B_decode], the slots of those rows as
 *                  pkv_slot_mapping gives them for the step (chunk rows
 *                  first); a negative slot writes nothing
 *   k_cache, v_cache   the pools, read and written (distinct)
 *   the other arguments as for pkv_attn_prefill_decode
 * Errors: those of pkv_attn_prefill_decode, and PKV_EINVAL for a null
 * k_new, v_new or slot_mapping or one pool for K and V.
 */
int pkv_attn_prefill_decode_append(
    void* out_prefill, const void* q_prefill, const int32_t* cu_q_lens,
    const int32_t* block_tables_prefill, const int32_t* context_lens_prefill, int32_t B_prefill,
    int32_t total_q, int32_t max_q_len, int32_t max_context_len_prefill, void* out_decode,
    const void* q_decode, const int32_t* block_tables_decode, const int32_t* context_lens_decode,
    int32_t B_decode, int32_t max_context_len_decode, const void* k_new, const void* v_new,
    const int32_t* slot_mapping, void* k_cache, void* v_cache, int32_t Hq, int32_t Hkv, int32_t D,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
    void* prefill_workspace, size_t prefill_workspace_bytes, void* decode_workspace,
    size_t decode_workspace_bytes, void* stream);

/*
 * The step before attention, fused ([P1] model.py: rms_norm, _rope_tables,
 * apply_rope and forward, which normalises q and k per head, rotates both at
 * the token's absolute position and writes k and v into the cache; the
 * pages name this fusion as the first one to write for the GPU).  For every
 * new token t of sequence b (cu_new_lens / context_lens as in
 * pkv_slot_mapping; position p = context_lens[b] - n_new_b + local index):
 *     q_out[t][h] = rope(rms_norm(q_in[t][h], q_norm_w), p)   for each query head h
 *     k_cache[slot][g] = rope(rms_norm(k_in[t][g], k_norm_w), p),  v_cache[slot][g] = v_in[t][g]
 * with rms_norm(x, w) = bf16(bf16(x * rsqrt(mean(x^2) + eps)) * w) (mean and
 * rsqrt in float32) and rope(x, p) = bf16(bf16(x * cos[p]) +
 * bf16(rotate_half(x) * sin[p])), rotate_half(x) = (-x[D/2:], x[:D/2]): the
 * listing's bf16 tensor arithmetic.  The slot is found from block_tables as
 * pkv_slot_mapping finds it and written to slot_mapping[t] (if not NULL; -1
 * when the table has no page there, or an entry outside [0, num_blocks) or
 * at least 2^27).  A token whose slot is -1 writes no
 * K/V; a position outside [0, max_pos) gives NaN q rows and writes no K/V.
 *   q_in, q_out     bf16 [T][Hq][D] (must not overlap)
 *   k_in, v_in      bf16 [T][Hkv][D]
 *   q_norm_w, k_norm_w  bf16 [D]
 *   cos_table, sin_table  bf16 [max_pos][D], both halves of a row equal
 *                   ([P1] _rope_tables: inv_freq = 1 / theta^(2i/D))
 *   k_cache, v_cache  the bf16 page pools ([num_blocks][16][Hkv][D], as pkv_append)
 * The only difference from the listing's arithmetic is the order of the
 * 128-term float32 sum of squares.
 */
int pkv_qk_norm_rope_append(void* q_out, const void* q_in, const void* k_in, const void* v_in,
                            const void* q_norm_w, const void* k_norm_w, const void* cos_table,
                            const void* sin_table, int32_t max_pos, const int32_t* block_tables,
                            const int32_t* cu_new_lens, const int32_t* context_lens,
                            int32_t* slot_mapping, void* k_cache, void* v_cache, int32_t B,
                            int32_t max_blocks_per_seq, int32_t T, int32_t num_blocks,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size, float eps,
                            void* stream);

/*
 * int8 KV pages ([P2] kv_cache.py listing, section 5, class KV8Cache: one
 * byte per element plus one float32 scale per (token, KV head); [P2] closing
 * notes: 2112 B instead of 4096 B per token-layer at H_kv 8, d_head 128).
 * Pool layout, the per-layer slice of KV8Cache's k, v [L, cap, H_kv, D] and
 * ks, vs [L, cap, H_kv] with cap cut into pages of 16 slots:
 *   k_codes, v_codes    int8 [num_blocks][16][Hkv][D], the order of the bf16
 *                       pools; a row of codes reads back as code * scale.
 *   k_scales, v_scales  float32 [num_blocks][Hkv][16]: the scale of the row
 *                       of (page b, slot s, KV head g) at [b][g][s].  Inside
 *                       a page the scales are head-major, so the 16 scales
 *                       one KV head reads from a page are one 64-byte run.
 * Unwritten slots may hold anything; a NaN scale there is never read.
 */

/*
 * int8 append ([P2] KV8Cache.write): every row x = k_new[t][g][:] (and the
 * V row) is quantised in float32 exactly as the page does,
 *     scale = max_d |x_d| / 127 + 1e-8,  code_d = clip(rint(x_d / scale), -127, 127)
 * (IEEE division, round half to even), and codes and scale are written to the
 * slot slot_mapping[t] of every KV head g; slots outside [0, num_blocks*16)
 * are skipped.  Inputs must be finite.  Slots must be distinct (duplicates
 * race; PKV_VALIDATE=1 rejects them).  D must be 128.
 *   k_new, v_new  bf16 [T][Hkv][D]
 */
int pkv_append_int8(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                    void* k_codes, void* v_codes, float* k_scales, float* v_scales, int32_t T,
                    int32_t num_blocks, int32_t Hkv, int32_t D, int32_t block_size, void* stream);

/*
 * Decode attention over int8 pages ([P2] KV8Cache.read: K and V read back as
 * code * scale, then the attention of pkv_attn_decode).  Same arguments,
 * outputs, error behaviour, split plan and workspace as pkv_attn_decode
 * (pkv_decode_workspace_bytes / pkv_decode_num_splits apply unchanged).
 * Scores use q . codes times the row's K scale; the row's V scale multiplies
 * its probability, which is rounded to bf16 for the PV product (bf16 weights
 * times codes, accumulated in float32).
 */
int pkv_attn_decode_int8(void* out, const void* q, const void* k_codes, const void* v_codes,
                         const float* k_scales, const float* v_scales,
                         const int32_t* block_tables,
                         const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                         int32_t D, int32_t block_size, int32_t num_blocks,
                         int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode over int8 pages with the step's append fused in ([P1] model.py
 * forward, as pkv_attn_decode_append; [P2] KV8Cache.write for the new rows):
 * position p = context_lens[b] - 1 of every sequence b takes k_new[b] /
 * v_new[b], quantised exactly as pkv_append_int8 quantises them (the same
 * codes and scale bits), and the call writes those codes and scales into the
 * slot of p (found from block_tables; nothing is written where there is
 * none), then attends as pkv_attn_decode_int8 with position p's codes taken
 * from registers.  The result equals pkv_append_int8 followed by
 * pkv_attn_decode_int8 up to the order of float32 sums.  One launch; no slot
 * mapping needed.  Same errors, split plan and workspace as
 * pkv_attn_decode_int8.
 *   k_new, v_new        bf16 [B][Hkv][D], the step's rows (finite)
 *   k_codes, v_codes    the int8 pools, read and written
 *   k_scales, v_scales  their scales, read and written
 */
int pkv_attn_decode_append_int8(void* out, const void* q, const void* k_new, const void* v_new,
                                void* k_codes, void* v_codes, float* k_scales, float* v_scales,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                                int32_t num_blocks, int32_t max_blocks_per_seq,
                                int32_t max_context_len, float scale, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Causal chunked prefill over int8 pages ([P2] KV8Cache.read: K and V read
 * back as code * scale; then the attention of pkv_attn_prefill_chunk).  Same
 * arguments, outputs, error behaviour, split plan and workspace as
 * pkv_attn_prefill_chunk (pkv_prefill_workspace_bytes applies unchanged),
 * with the pools replaced by k_codes, v_codes, k_scales and v_scales in the
 * layout above.  Each tile of 64 keys is dequantised once per workgroup, code *
 * scale rounded to bf16, and the bf16 MFMA path runs on the result.
 */
int pkv_attn_prefill_chunk_int8(void* out, const void* q, const int32_t* cu_q_lens,
                                const void* k_codes, const void* v_codes, const float* k_scales,
                                const float* v_scales,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int32_t B, int32_t total_q, int32_t max_q_len, int32_t Hq,
                                int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * The attention of a mixed step over int8 pages ([P1] "Why chunked prefill";
 * [P2] KV8Cache.read): pkv_attn_prefill_chunk_int8 over the prefill
 * sequences and pkv_attn_decode_int8 over the decode sequences, with the same
 * outputs bit for bit, as pkv_attn_prefill_decode does for bf16 pages.
 * Group sizes 1, 2 and 4 run as one launch holding both kinds of workgroup
 * (one per compute unit: the chunk's code ring takes most of the LDS); group
 * size 8, or one half empty, runs the two launches in order.  Arguments as
 * for pkv_attn_prefill_decode, with the pools replaced by k_codes, v_codes,
 * k_scales and v_scales in the layout above.  Errors: those of
 * pkv_attn_prefill_decode, and PKV_EINVAL for null scales.  The step's rows
 * must be appended (pkv_append_int8) before the call.
 */
int pkv_attn_prefill_decode_int8(
    void* out_prefill, const void* q_prefill, const int32_t* cu_q_lens,
    const int32_t* block_tables_prefill, const int32_t* context_lens_prefill, int32_t B_prefill,
    int32_t total_q, int32_t max_q_len, int32_t max_context_len_prefill, void* out_decode,
    const void* q_decode, const int32_t* block_tables_decode, const int32_t* context_lens_decode,
    int32_t B_decode, int32_t max_context_len_decode, const void* k_codes, const void* v_codes,
    const float* k_scales, const float* v_scales, int32_t Hq, int32_t Hkv, int32_t D,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
    void* prefill_workspace, size_t prefill_workspace_bytes, void* decode_workspace,
    size_t decode_workspace_bytes, void* stream);

/*
 * Ring (sliding-window) paging ([P2] section 4, "Capacity-cache": beyond the
 * capacity the cache becomes a ring, position p is written at index
 * p % capacity over the oldest token, a read returns the last
 * min(end, capacity) positions with their absolute positions, and the causal
 * mask compares absolute positions; [P2] kv_cache.py listing,
 * KVCache.write/read).  A sequence's ring of `window` tokens (a positive
 * multiple of 16, at most max_blocks_per_seq * 16) is the first window / 16
 * pages of its table: position p lives at page (p % window) / 16, offset
 * p % 16.  context_lens count every position written so far and may exceed
 * the table.  Each call below behaves as its non-ring counterpart except:
 *   pkv_slot_mapping_ring       slots of positions p at ring index p % window;
 *   pkv_attn_decode_ring        the query attends to the ring's min(n, window)
 *                               keys (a sliding window of `window` tokens);
 *                               workspace: pkv_decode_workspace_bytes(B, Hq,
 *                               Hkv, D, min(max_context_len, window));
 *   pkv_attn_prefill_chunk_ring the chunk is in the ring already; row t at
 *                               position n - T + t attends to the ring's keys
 *                               at positions max(0, n - window) .. its own;
 *                               max_q_len <= window; workspace:
 *                               pkv_prefill_workspace_bytes(B, max_q_len, Hq,
 *                               Hkv, D, min(max_context_len, window + 64)).
 */
int pkv_slot_mapping_ring(int32_t* slot_mapping, const int32_t* block_tables,
                          const int32_t* cu_new_lens, const int32_t* context_lens, int32_t B,
                          int32_t max_blocks_per_seq, int32_t total_new, int32_t block_size,
                          int32_t window, void* stream);

/* Decode over rings ([P2] section 4): the query at position n - 1 attends to
 * the last min(n, window) positions, all held by the ring. */
int pkv_attn_decode_ring(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                         int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                         int32_t window, float scale, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Causal chunk over rings ([P2] section 4 and KVCache.read: the chunk is
 * written first; its rows see the ring's keys at or before their position). */
int pkv_attn_prefill_chunk_ring(void* out, const void* q, const int32_t* cu_q_lens,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int32_t B, int32_t total_q, int32_t max_q_len, int32_t Hq,
                                int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_context_len,
                                int32_t window, float scale, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Thread-local message describing the last non-OK return on this thread. */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
