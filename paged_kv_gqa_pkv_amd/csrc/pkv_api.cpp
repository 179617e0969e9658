// C ABI of the paged GQA attention library: argument checks, split planning,
// launches, thread-local error strings.  No allocation, no device->host sync
// (except under PKV_VALIDATE=1, a debug mode that inspects index contents).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_set>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
}

bool validate_mode() {
  static const bool on = [] {
    const char* v = std::getenv("PKV_VALIDATE");
    return v && v[0] && std::strcmp(v, "0") != 0;
  }();
  return on;
}

// Compute units of the current device, cached per device id.
int device_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

int check_geometry(int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size) {
  if (Hq <= 0 || Hkv <= 0 || D <= 0 || block_size <= 0)
    return fail(PKV_EINVAL, "head counts, head_dim and block_size must be positive");
  if (block_size != PKV_BLOCK_SIZE)
    return fail(PKV_EUNSUPPORTED, "block_size %d unsupported (pages hold 16 tokens)", block_size);
  if (D != PKV_HEAD_DIM) return fail(PKV_EUNSUPPORTED, "head_dim %d unsupported (only 128)", D);
  if (Hq % Hkv) return fail(PKV_EUNSUPPORTED, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PKV_EUNSUPPORTED, "group size Hq/Hkv=%d unsupported (1, 2, 4 or 8)", G);
  return PKV_OK;
}

template <typename T>
bool to_host(std::vector<T>& dst, const T* src, size_t n, hipStream_t stream) {
  dst.resize(n);
  if (n == 0) return true;
  if (hipStreamSynchronize(stream) != hipSuccess) return false;
  return hipMemcpy(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost) == hipSuccess;
}

// PKV_VALIDATE: block tables and lengths of a decode/prefill call.
int validate_tables(const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                    int32_t max_blocks, int32_t num_blocks, int32_t max_context_len,
                    hipStream_t stream, int32_t window = 0) {
  std::vector<int32_t> ctx, bt;
  if (!to_host(ctx, context_lens, (size_t)B, stream) ||
      !to_host(bt, block_tables, (size_t)B * max_blocks, stream))
    return fail(PKV_ELAUNCH, "PKV_VALIDATE: copy of index arrays failed");
  for (int b = 0; b < B; ++b) {
    const int n = ctx[b];
    if (n < 0 || n > max_context_len)
      return fail(PKV_EVALIDATE, "context_lens[%d]=%d outside [0, max_context_len=%d]", b, n,
                  max_context_len);
    if (window == 0 && (int64_t)n > (int64_t)max_blocks * PKV_BLOCK_SIZE)
      return fail(PKV_EVALIDATE, "context_lens[%d]=%d exceeds the table (%d pages)", b, n,
                  max_blocks);
    const int used = window > 0 && n > window ? window : n;   // a ring uses its first pages
    for (int i = 0; i < (used + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE; ++i) {
      const int blk = bt[(size_t)b * max_blocks + i];
      if (blk < 0 || blk >= num_blocks)
        return fail(PKV_EVALIDATE, "block_tables[%d][%d]=%d outside [0, %d)", b, i, blk,
                    num_blocks);
    }
  }
  return PKV_OK;
}

// PKV_VALIDATE: every slot inside the pool and no slot twice.
int validate_slots(const int32_t* slot_mapping, int32_t T, int32_t num_blocks, hipStream_t s) {
  std::vector<int32_t> slots;
  if (!to_host(slots, slot_mapping, (size_t)T, s))
    return fail(PKV_ELAUNCH, "PKV_VALIDATE: copy of slot_mapping failed");
  std::unordered_set<int32_t> seen;
  for (int t = 0; t < T; ++t) {
    const int32_t v = slots[t];
    if (v < 0) continue;
    if ((int64_t)v >= (int64_t)num_blocks * PKV_BLOCK_SIZE)
      return fail(PKV_EVALIDATE, "slot_mapping[%d]=%d outside a pool of %d pages", t, v,
                  num_blocks);
    if (!seen.insert(v).second)
      return fail(PKV_EVALIDATE, "slot %d appears twice in slot_mapping", v);
  }
  return PKV_OK;
}

// A ring of `window` tokens: a positive multiple of the page size that fits the table.
// Positions and slots are int32, so a block table row is at most 2^27 - 1
// pages wide (its token count, width * 16, then fits in int32).
int check_table_width(int32_t max_blocks_per_seq) {
  if (max_blocks_per_seq >= (1 << 27))
    return fail(PKV_EINVAL, "max_blocks_per_seq=%d: a table row holds at most 2^27 - 1 pages",
                max_blocks_per_seq);
  return PKV_OK;
}

int check_window(int32_t window, int32_t max_blocks_per_seq) {
  if (window <= 0 || window % PKV_BLOCK_SIZE)
    return fail(PKV_EINVAL, "window=%d must be a positive multiple of %d", window, PKV_BLOCK_SIZE);
  if ((int64_t)window > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE)
    return fail(PKV_EINVAL, "window=%d exceeds the block table (%d pages)", window,
                max_blocks_per_seq);
  return PKV_OK;
}

// Host checks shared by the decode entry points; fills the split plan.
// done = true: nothing to launch (B == 0).  own_buffers: the split buffers
// are the library's array (checked by the caller), not `workspace`.
int check_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* context_lens, int32_t B, int32_t Hq,
                 int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                 int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                 void* workspace, size_t workspace_bytes, void* stream, pkv::DecodePlan& plan,
                 bool& done, int32_t window = 0, bool own_buffers = false) {
  done = false;
  if (B < 0 || num_blocks < 0 || max_blocks_per_seq < 0 || max_context_len < 0)
    return fail(PKV_EINVAL, "negative size");
  if (check_table_width(max_blocks_per_seq)) return PKV_EINVAL;
  int rc = check_geometry(Hq, Hkv, D, block_size);
  if (rc) return rc;
  if (B == 0) { done = true; return PKV_OK; }
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_EINVAL, "null pointer argument");
  if (out == q) return fail(PKV_EINVAL, "out and q must not overlap");
  if (window > 0) {
    rc = check_window(window, max_blocks_per_seq);
    if (rc) return rc;
  } else if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE) {
    return fail(PKV_EINVAL, "max_context_len=%d exceeds the block table (%d pages)",
                max_context_len, max_blocks_per_seq);
  }
  if (!(scale == scale)) return fail(PKV_EINVAL, "scale is NaN");
  const int32_t plan_ctx = window > 0 && max_context_len > window ? window : max_context_len;
  plan = pkv::plan_decode(B, Hq, Hkv, plan_ctx, device_cus());
  if (!own_buffers && (plan.ws_bytes > workspace_bytes || (plan.ws_bytes && !workspace)))
    return fail(PKV_EWORKSPACE, "decode needs %zu workspace bytes, got %zu", plan.ws_bytes,
                workspace_bytes);
  if (own_buffers && !pkv::noalloc_fits(plan, B, Hkv))
    return fail(PKV_EWORKSPACE,
                "decode of this shape needs %zu bytes of split buffers (%d counters); the "
                "library's array holds %d bytes (%d counters): use pkv_attn_decode with a "
                "workspace",
                plan.ws_bytes, B * Hkv, (int)PKV_NOALLOC_SCRATCH_BYTES,
                (int)(PKV_NOALLOC_COUNTER_BYTES / sizeof(int)));
  if (validate_mode()) {
    rc = validate_tables(block_tables, context_lens, B, max_blocks_per_seq, num_blocks,
                         max_context_len, static_cast<hipStream_t>(stream), window);
    if (rc) return rc;
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_err; }

const char* pkv_version(void) { return "pkv 0.1 gfx950"; }

static int slot_mapping_impl(int32_t* slot_mapping, const int32_t* block_tables,
                             const int32_t* cu_new_lens, const int32_t* context_lens, int32_t B,
                             int32_t max_blocks_per_seq, int32_t total_new, int32_t block_size,
                             int32_t window, void* stream) {
  if (B < 0 || total_new < 0 || max_blocks_per_seq < 0)
    return fail(PKV_EINVAL, "negative size");
  if (check_table_width(max_blocks_per_seq)) return PKV_EINVAL;
  if (block_size != PKV_BLOCK_SIZE)
    return fail(PKV_EUNSUPPORTED, "block_size %d unsupported (pages hold 16 tokens)", block_size);
  if (total_new == 0) return PKV_OK;
  if (B == 0) return fail(PKV_EINVAL, "total_new=%d tokens but no sequences", total_new);
  if (window > 0) {
    const int rc = check_window(window, max_blocks_per_seq);
    if (rc) return rc;
  }
  if (!slot_mapping || !block_tables || !cu_new_lens || !context_lens)
    return fail(PKV_EINVAL, "null pointer argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_mode()) {
    std::vector<int32_t> cu, ctx;
    if (!to_host(cu, cu_new_lens, (size_t)B + 1, s) || !to_host(ctx, context_lens, (size_t)B, s))
      return fail(PKV_ELAUNCH, "PKV_VALIDATE: copy of index arrays failed");
    if (cu[0] != 0 || cu[B] != total_new)
      return fail(PKV_EVALIDATE, "cu_new_lens must start at 0 and end at total_new=%d", total_new);
    for (int b = 0; b < B; ++b) {
      if (cu[b + 1] < cu[b]) return fail(PKV_EVALIDATE, "cu_new_lens decreases at %d", b);
      if (cu[b + 1] - cu[b] > ctx[b])
        return fail(PKV_EVALIDATE, "sequence %d appends %d tokens but its context is %d", b,
                    cu[b + 1] - cu[b], ctx[b]);
      if (window == 0 && (int64_t)ctx[b] > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE)
        return fail(PKV_EVALIDATE, "context_lens[%d]=%d exceeds the table", b, ctx[b]);
    }
  }
  return launch_status(pkv::launch_slot_mapping(slot_mapping, block_tables, cu_new_lens,
                                                context_lens, B, max_blocks_per_seq, total_new,
                                                window, s),
                       "pkv_slot_mapping");
}

int pkv_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables,
                     const int32_t* cu_new_lens, const int32_t* context_lens, int32_t B,
                     int32_t max_blocks_per_seq, int32_t total_new, int32_t block_size,
                     void* stream) {
  return slot_mapping_impl(slot_mapping, block_tables, cu_new_lens, context_lens, B,
                           max_blocks_per_seq, total_new, block_size, 0, stream);
}

int pkv_slot_mapping_ring(int32_t* slot_mapping, const int32_t* block_tables,
                          const int32_t* cu_new_lens, const int32_t* context_lens, int32_t B,
                          int32_t max_blocks_per_seq, int32_t total_new, int32_t block_size,
                          int32_t window, void* stream) {
  if (window <= 0) return fail(PKV_EINVAL, "window=%d must be positive", window);
  return slot_mapping_impl(slot_mapping, block_tables, cu_new_lens, context_lens, B,
                           max_blocks_per_seq, total_new, block_size, window, stream);
}


int pkv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping, void* k_cache,
               void* v_cache, int32_t T, int32_t num_blocks, int32_t Hkv, int32_t D,
               int32_t block_size, void* stream) {
  if (T < 0 || num_blocks < 0) return fail(PKV_EINVAL, "negative size");
  int rc = check_geometry(Hkv, Hkv, D, block_size);
  if (rc) return rc;
  if (T == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache)
    return fail(PKV_EINVAL, "null pointer argument");
  if (k_cache == v_cache) return fail(PKV_EINVAL, "k_cache and v_cache must differ");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_mode()) {
    rc = validate_slots(slot_mapping, T, num_blocks, s);
    if (rc) return rc;
  }
  return launch_status(
      pkv::launch_append(k_new, v_new, slot_mapping, k_cache, v_cache, T, num_blocks, Hkv, D, s),
      "pkv_append");
}

int pkv_append_int8(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                    void* k_codes, void* v_codes, float* k_scales, float* v_scales, int32_t T,
                    int32_t num_blocks, int32_t Hkv, int32_t D, int32_t block_size, void* stream) {
  if (T < 0 || num_blocks < 0) return fail(PKV_EINVAL, "negative size");
  int rc = check_geometry(Hkv, Hkv, D, block_size);
  if (rc) return rc;
  if (T == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_codes || !v_codes || !k_scales || !v_scales)
    return fail(PKV_EINVAL, "null pointer argument");
  if (k_codes == v_codes) return fail(PKV_EINVAL, "k_codes and v_codes must differ");
  if (k_scales == v_scales) return fail(PKV_EINVAL, "k_scales and v_scales must differ");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_mode()) {
    rc = validate_slots(slot_mapping, T, num_blocks, s);
    if (rc) return rc;
  }
  return launch_status(pkv::launch_append_int8(k_new, v_new, slot_mapping, k_codes, v_codes,
                                               k_scales, v_scales, T, num_blocks, Hkv, D, s),
                       "pkv_append_int8");
}

int pkv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src_blocks,
                    const int32_t* dst_blocks, int32_t n_pairs, int32_t num_blocks,
                    int64_t block_bytes, int32_t n_layers, int64_t layer_stride_bytes,
                    void* stream) {
  if (n_pairs < 0 || num_blocks < 0 || block_bytes < 0 || n_layers < 0 || layer_stride_bytes < 0)
    return fail(PKV_EINVAL, "negative size");
  if (n_pairs == 0 || n_layers == 0 || block_bytes == 0) return PKV_OK;
  if (!k_pool || !src_blocks || !dst_blocks) return fail(PKV_EINVAL, "null pointer argument");
  if (k_pool == v_pool) return fail(PKV_EINVAL, "k_pool and v_pool must differ");
  if (block_bytes % 16 || layer_stride_bytes % 16 || (uintptr_t)k_pool % 16 ||
      (uintptr_t)v_pool % 16)
    return fail(PKV_EINVAL, "pools, block_bytes and layer_stride_bytes must be 16-byte aligned");
  if (n_layers > 1 && layer_stride_bytes < (int64_t)num_blocks * block_bytes)
    return fail(PKV_EINVAL, "layer_stride_bytes=%lld is smaller than a layer's %d blocks",
                (long long)layer_stride_bytes, num_blocks);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_mode()) {
    std::vector<int32_t> src, dst;
    if (!to_host(src, src_blocks, (size_t)n_pairs, s) || !to_host(dst, dst_blocks, (size_t)n_pairs, s))
      return fail(PKV_ELAUNCH, "PKV_VALIDATE: copy of the block pairs failed");
    std::unordered_set<int32_t> srcs(src.begin(), src.end()), dsts;
    for (int i = 0; i < n_pairs; ++i) {
      if (src[i] < 0 || src[i] >= num_blocks || dst[i] < 0 || dst[i] >= num_blocks)
        return fail(PKV_EVALIDATE, "pair %d (%d -> %d) outside a pool of %d blocks", i, src[i],
                    dst[i], num_blocks);
      if (!dsts.insert(dst[i]).second)
        return fail(PKV_EVALIDATE, "block %d is a destination twice", dst[i]);
      if (srcs.count(dst[i]))
        return fail(PKV_EVALIDATE, "block %d is both a source and a destination", dst[i]);
    }
  }
  return launch_status(pkv::launch_copy_blocks(k_pool, v_pool, src_blocks, dst_blocks, n_pairs,
                                               num_blocks, block_bytes, n_layers,
                                               layer_stride_bytes, s),
                       "pkv_copy_blocks");
}

int pkv_qk_norm_rope_append(void* q_out, const void* q_in, const void* k_in, const void* v_in,
                            const void* q_norm_w, const void* k_norm_w, const void* cos_table,
                            const void* sin_table, int32_t max_pos, const int32_t* block_tables,
                            const int32_t* cu_new_lens, const int32_t* context_lens,
                            int32_t* slot_mapping, void* k_cache, void* v_cache, int32_t B,
                            int32_t max_blocks_per_seq, int32_t T, int32_t num_blocks,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size, float eps,
                            void* stream) {
  if (B < 0 || T < 0 || num_blocks < 0 || max_blocks_per_seq < 0 || max_pos < 0)
    return fail(PKV_EINVAL, "negative size");
  if (check_table_width(max_blocks_per_seq)) return PKV_EINVAL;
  int rc = check_geometry(Hq, Hkv, D, block_size);
  if (rc) return rc;
  if (T == 0) return PKV_OK;
  if (B == 0) return fail(PKV_EINVAL, "T=%d tokens but no sequences", T);
  if (!q_out || !q_in || !k_in || !v_in || !q_norm_w || !k_norm_w || !cos_table || !sin_table ||
      !block_tables || !cu_new_lens || !context_lens || !k_cache || !v_cache)
    return fail(PKV_EINVAL, "null pointer argument");
  if (q_out == q_in) return fail(PKV_EINVAL, "q_out and q_in must not overlap");
  if (k_cache == v_cache) return fail(PKV_EINVAL, "k_cache and v_cache must differ");
  if (!(eps >= 0.f)) return fail(PKV_EINVAL, "eps must be >= 0");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_mode()) {
    std::vector<int32_t> cu, ctx;
    if (!to_host(cu, cu_new_lens, (size_t)B + 1, s) || !to_host(ctx, context_lens, (size_t)B, s))
      return fail(PKV_ELAUNCH, "PKV_VALIDATE: copy of index arrays failed");
    if (cu[0] != 0 || cu[B] != T)
      return fail(PKV_EVALIDATE, "cu_new_lens must start at 0 and end at T=%d", T);
    for (int b = 0; b < B; ++b) {
      if (cu[b + 1] < cu[b] || cu[b + 1] - cu[b] > ctx[b])
        return fail(PKV_EVALIDATE, "sequence %d: inconsistent cu_new_lens / context_lens", b);
      if (ctx[b] > max_pos)
        return fail(PKV_EVALIDATE, "context_lens[%d]=%d beyond the RoPE tables (%d rows)", b,
                    ctx[b], max_pos);
    }
    rc = validate_tables(block_tables, context_lens, B, max_blocks_per_seq, num_blocks,
                         max_blocks_per_seq * PKV_BLOCK_SIZE, s);
    if (rc) return rc;
  }
  return launch_status(pkv::launch_qk_norm_rope_append(
                           q_out, q_in, k_in, v_in, q_norm_w, k_norm_w, cos_table, sin_table,
                           max_pos, block_tables, cu_new_lens, context_lens, slot_mapping,
                           k_cache, v_cache, B, max_blocks_per_seq, T, num_blocks, Hq, Hkv, eps,
                           s),
                       "pkv_qk_norm_rope_append");
}

size_t pkv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t max_context_len) {
  if (B <= 0 || max_context_len < 0 || check_geometry(Hq, Hkv, D, PKV_BLOCK_SIZE) != PKV_OK)
    return 0;
  return pkv::plan_decode(B, Hq, Hkv, max_context_len, device_cus()).ws_bytes;
}

int32_t pkv_decode_num_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                              int32_t max_context_len) {
  if (B <= 0 || max_context_len < 0 || check_geometry(Hq, Hkv, D, PKV_BLOCK_SIZE) != PKV_OK)
    return 1;
  return pkv::plan_decode(B, Hq, Hkv, max_context_len, device_cus()).splits;
}

int pkv_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                    int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                    int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
  pkv::DecodePlan plan;
  bool done = false;
  int rc = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, D,
                        block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                        workspace, workspace_bytes, stream, plan, done);
  if (rc || done) return rc;
  return launch_status(pkv::launch_decode(out, q, k_cache, v_cache, block_tables, context_lens, B,
                                          Hq, Hkv, num_blocks, max_blocks_per_seq, scale, 0, plan,
                                          workspace, static_cast<hipStream_t>(stream)),
                       "pkv_attn_decode");
}

int pkv_attn_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                           void* k_cache, void* v_cache, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t block_size, int32_t num_blocks,
                           int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                           void* workspace, size_t workspace_bytes, void* stream) {
  pkv::DecodePlan plan;
  bool done = false;
  int rc = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, D,
                        block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                        workspace, workspace_bytes, stream, plan, done);
  if (rc || done) return rc;
  if (!k_new || !v_new) return fail(PKV_EINVAL, "null pointer argument");
  if (k_cache == v_cache) return fail(PKV_EINVAL, "k_cache and v_cache must differ");
  return launch_status(pkv::launch_decode_append(out, q, k_new, v_new, k_cache, v_cache,
                                                 block_tables, context_lens, B, Hq, Hkv,
                                                 num_blocks, max_blocks_per_seq, scale, plan,
                                                 workspace, static_cast<hipStream_t>(stream)),
                       "pkv_attn_decode_append");
}

int pkv_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                            int32_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t max_context_len, float scale, void* stream) {
  pkv::DecodePlan plan;
  bool done = false;
  const int rc = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv,
                              D, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                              scale, nullptr, 0, stream, plan, done, 0, true);
  if (rc || done) return rc;
  return launch_status(pkv::launch_decode_noalloc(out, q, k_cache, v_cache, block_tables,
                                                  context_lens, B, Hq, Hkv, num_blocks,
                                                  max_blocks_per_seq, scale, plan,
                                                  static_cast<hipStream_t>(stream)),
                       "pkv_attn_decode_noalloc");
}

int pkv_attn_decode_ring(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                         int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                         int32_t window, float scale, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (window <= 0) return fail(PKV_EINVAL, "window=%d must be positive", window);
  pkv::DecodePlan plan;
  bool done = false;
  int rc = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, D,
                        block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                        workspace, workspace_bytes, stream, plan, done, window);
  if (rc || done) return rc;
  return launch_status(pkv::launch_decode(out, q, k_cache, v_cache, block_tables, context_lens, B,
                                          Hq, Hkv, num_blocks, max_blocks_per_seq, scale, window,
                                          plan, workspace, static_cast<hipStream_t>(stream)),
                       "pkv_attn_decode_ring");
}

int pkv_attn_decode_append_int8(void* out, const void* q, const void* k_new, const void* v_new,
                                void* k_codes, void* v_codes, float* k_scales, float* v_scales,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                                int32_t num_blocks, int32_t max_blocks_per_seq,
                                int32_t max_context_len, float scale, void* workspace,
                                size_t workspace_bytes, void* stream) {
  pkv::DecodePlan plan;
  bool done = false;
  if (B > 0 && (!k_scales || !v_scales)) return fail(PKV_EINVAL, "null pointer argument");
  int rc = check_decode(out, q, k_codes, v_codes, block_tables, context_lens, B, Hq, Hkv, D,
                        block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                        workspace, workspace_bytes, stream, plan, done);
  if (rc || done) return rc;
  if (!k_new || !v_new) return fail(PKV_EINVAL, "null pointer argument");
  if (k_codes == v_codes) return fail(PKV_EINVAL, "k_codes and v_codes must differ");
  if (k_scales == v_scales) return fail(PKV_EINVAL, "k_scales and v_scales must differ");
  return launch_status(pkv::launch_decode_append_int8(out, q, k_new, v_new, k_codes, v_codes,
                                                      k_scales, v_scales, block_tables,
                                                      context_lens, B, Hq, Hkv, num_blocks,
                                                      max_blocks_per_seq, scale, plan, workspace,
                                                      static_cast<hipStream_t>(stream)),
                       "pkv_attn_decode_append_int8");
}

int pkv_attn_decode_int8(void* out, const void* q, const void* k_codes, const void* v_codes,
                         const float* k_scales, const float* v_scales,
                         const int32_t* block_tables,
                         const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                         int32_t D, int32_t block_size, int32_t num_blocks,
                         int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                         void* workspace, size_t workspace_bytes, void* stream) {
  pkv::DecodePlan plan;
  bool done = false;
  if (B > 0 && (!k_scales || !v_scales)) return fail(PKV_EINVAL, "null pointer argument");
  int rc = check_decode(out, q, k_codes, v_codes, block_tables, context_lens, B, Hq, Hkv, D,
                        block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                        workspace, workspace_bytes, stream, plan, done);
  if (rc || done) return rc;
  return launch_status(pkv::launch_decode_int8(out, q, k_codes, v_codes, k_scales, v_scales,
                                               block_tables,
                                               context_lens, B, Hq, Hkv, num_blocks,
                                               max_blocks_per_seq, scale, plan, workspace,
                                               static_cast<hipStream_t>(stream)),
                       "pkv_attn_decode_int8");
}

size_t pkv_prefill_workspace_bytes(int32_t B, int32_t max_q_len, int32_t Hq, int32_t Hkv,
                                   int32_t D, int32_t max_context_len) {
  if (B <= 0 || max_q_len <= 0 || max_context_len < 0 ||
      check_geometry(Hq, Hkv, D, PKV_BLOCK_SIZE) != PKV_OK)
    return 0;
  return pkv::plan_prefill(B, max_q_len, Hq, Hkv, max_context_len, device_cus()).ws_bytes;
}

// Host checks shared by the chunked-prefill entry points; fills the
// key-split plan.  done = true: nothing to launch.
static int check_prefill(void* out, const void* q, const int32_t* cu_q_lens,
                         const void* k_cache, const void* v_cache,
                         const int32_t* block_tables,
                         const int32_t* context_lens, int32_t B, int32_t total_q,
                         int32_t max_q_len, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                         int32_t max_context_len, int32_t window, float scale, void* workspace,
                         size_t workspace_bytes, void* stream, pkv::PrefillPlan& plan,
                         bool& done) {
  done = true;
  if (B < 0 || total_q < 0 || max_q_len < 0 || num_blocks < 0 || max_blocks_per_seq < 0 ||
      max_context_len < 0)
    return fail(PKV_EINVAL, "negative size");
  if (check_table_width(max_blocks_per_seq)) return PKV_EINVAL;
  int rc = check_geometry(Hq, Hkv, D, block_size);
  if (rc) return rc;
  if (B == 0 || total_q == 0) return PKV_OK;
  if (!out || !q || !cu_q_lens || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_EINVAL, "null pointer argument");
  if (out == q) return fail(PKV_EINVAL, "out and q must not overlap");
  if (max_q_len > total_q) return fail(PKV_EINVAL, "max_q_len=%d > total_q=%d", max_q_len, total_q);
  if (window > 0) {
    rc = check_window(window, max_blocks_per_seq);
    if (rc) return rc;
    if (max_q_len > window)
      return fail(PKV_EINVAL, "max_q_len=%d exceeds the ring of %d tokens", max_q_len, window);
  } else if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE) {
    return fail(PKV_EINVAL, "max_context_len=%d exceeds the block table (%d pages)",
                max_context_len, max_blocks_per_seq);
  }
  if (!(scale == scale)) return fail(PKV_EINVAL, "scale is NaN");
  if (max_q_len == 0) return PKV_OK;
  // A ring's keys span at most window positions, i.e. window / 64 + 1 key tiles.
  const int32_t plan_ctx =
      window > 0 && max_context_len > window + 64 ? window + 64 : max_context_len;
  plan = pkv::plan_prefill(B, max_q_len, Hq, Hkv, plan_ctx, device_cus());
  if (!plan.ok)
    return fail(PKV_EUNSUPPORTED, "max_context_len=%d exceeds the prefill kernel's 131072 keys",
                max_context_len);
  if (plan.ws_bytes > workspace_bytes || (plan.ws_bytes && !workspace))
    return fail(PKV_EWORKSPACE, "prefill needs %zu workspace bytes, got %zu", plan.ws_bytes,
                workspace_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_mode()) {
    std::vector<int32_t> cu, ctx;
    if (!to_host(cu, cu_q_lens, (size_t)B + 1, s) || !to_host(ctx, context_lens, (size_t)B, s))
      return fail(PKV_ELAUNCH, "PKV_VALIDATE: copy of index arrays failed");
    if (cu[0] != 0 || cu[B] != total_q)
      return fail(PKV_EVALIDATE, "cu_q_lens must start at 0 and end at total_q=%d", total_q);
    for (int b = 0; b < B; ++b) {
      const int T = cu[b + 1] - cu[b];
      if (T < 0 || T > max_q_len)
        return fail(PKV_EVALIDATE, "sequence %d has %d query rows (max_q_len=%d)", b, T,
                    max_q_len);
      if (T > ctx[b])
        return fail(PKV_EVALIDATE, "sequence %d has %d query rows but context %d", b, T, ctx[b]);
    }
    rc = validate_tables(block_tables, context_lens, B, max_blocks_per_seq, num_blocks,
                         max_context_len, s, window);
    if (rc) return rc;
  }
  done = false;
  return PKV_OK;
}

static int prefill_impl(void* out, const void* q, const int32_t* cu_q_lens,
                        const void* k_cache, const void* v_cache, const float* k_scales,
                        const float* v_scales,
                        const int32_t* block_tables,
                        const int32_t* context_lens, int32_t B, int32_t total_q,
                        int32_t max_q_len, int32_t Hq, int32_t Hkv, int32_t D,
                        int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                        int32_t max_context_len, int32_t window, float scale, void* workspace,
                        size_t workspace_bytes, void* stream) {
  pkv::PrefillPlan plan;
  bool done = true;
  const int rc = check_prefill(out, q, cu_q_lens, k_cache, v_cache, block_tables, context_lens,
                               B, total_q, max_q_len, Hq, Hkv, D, block_size, num_blocks,
                               max_blocks_per_seq, max_context_len, window, scale, workspace,
                               workspace_bytes, stream, plan, done);
  if (rc || done) return rc;
  return launch_status(pkv::launch_prefill(out, q, cu_q_lens, k_cache, v_cache, k_scales, v_scales,
                                           block_tables, context_lens, B, total_q, max_q_len, Hq,
                                           Hkv, num_blocks, max_blocks_per_seq, scale, window,
                                           plan, workspace, static_cast<hipStream_t>(stream)),
                       k_scales ? "pkv_attn_prefill_chunk_int8" : "pkv_attn_prefill_chunk");
}

int pkv_attn_prefill_chunk(void* out, const void* q, const int32_t* cu_q_lens,
                           const void* k_cache, const void* v_cache, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t B, int32_t total_q,
                           int32_t max_q_len, int32_t Hq, int32_t Hkv, int32_t D,
                           int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                           int32_t max_context_len, float scale, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return prefill_impl(out, q, cu_q_lens, k_cache, v_cache, nullptr, nullptr, block_tables,
                      context_lens, B, total_q, max_q_len, Hq, Hkv, D, block_size, num_blocks,
                      max_blocks_per_seq, max_context_len, 0, scale, workspace, workspace_bytes,
                      stream);
}

int pkv_attn_prefill_chunk_ring(void* out, const void* q, const int32_t* cu_q_lens,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int32_t B, int32_t total_q, int32_t max_q_len, int32_t Hq,
                                int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_context_len,
                                int32_t window, float scale, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (window <= 0) return fail(PKV_EINVAL, "window=%d must be positive", window);
  return prefill_impl(out, q, cu_q_lens, k_cache, v_cache, nullptr, nullptr, block_tables,
                      context_lens, B, total_q, max_q_len, Hq, Hkv, D, block_size, num_blocks,
                      max_blocks_per_seq, max_context_len, window, scale, workspace,
                      workspace_bytes, stream);
}

int pkv_attn_prefill_chunk_int8(void* out, const void* q, const int32_t* cu_q_lens,
                                const void* k_codes, const void* v_codes, const float* k_scales,
                                const float* v_scales,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int32_t B, int32_t total_q, int32_t max_q_len, int32_t Hq,
                                int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (B > 0 && total_q > 0 && (!k_scales || !v_scales))
    return fail(PKV_EINVAL, "null pointer argument");
  return prefill_impl(out, q, cu_q_lens, k_codes, v_codes, k_scales, v_scales, block_tables,
                      context_lens, B, total_q, max_q_len, Hq, Hkv, D, block_size, num_blocks,
                      max_blocks_per_seq, max_context_len, 0, scale, workspace, workspace_bytes,
                      stream);
}

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
                            void* stream) {
  pkv::PrefillPlan pplan;
  bool pdone = true;
  int rc = check_prefill(out_prefill, q_prefill, cu_q_lens, k_cache, v_cache,
                         block_tables_prefill, context_lens_prefill, B_prefill, total_q,
                         max_q_len, Hq, Hkv, D, block_size, num_blocks, max_blocks_per_seq,
                         max_context_len_prefill, 0, scale, prefill_workspace,
                         prefill_workspace_bytes, stream, pplan, pdone);
  if (rc) return rc;
  pkv::DecodePlan dplan;
  bool ddone = false;
  rc = check_decode(out_decode, q_decode, k_cache, v_cache, block_tables_decode,
                    context_lens_decode, B_decode, Hq, Hkv, D, block_size, num_blocks,
                    max_blocks_per_seq, max_context_len_decode, scale, decode_workspace,
                    decode_workspace_bytes, stream, dplan, ddone);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!pdone && !ddone) {
    if (out_prefill == out_decode) return fail(PKV_EINVAL, "the two outputs must differ");
    if (pplan.ws_bytes && dplan.ws_bytes && prefill_workspace == decode_workspace)
      return fail(PKV_EINVAL, "the two workspaces must differ");
    if (pkv::mixed_plan_fits(dplan, Hq / Hkv))
      return launch_status(
          pkv::launch_prefill_decode(out_prefill, q_prefill, cu_q_lens, block_tables_prefill,
                                     context_lens_prefill, B_prefill, total_q, max_q_len, pplan,
                                     prefill_workspace, out_decode, q_decode,
                                     block_tables_decode, context_lens_decode, B_decode, dplan,
                                     decode_workspace, k_cache, v_cache, Hq, Hkv, num_blocks,
                                     max_blocks_per_seq, scale, s),
          "pkv_attn_prefill_decode");
  }
  // one half only, or a shape the one-grid launch does not take: the two
  // launches one after the other
  if (!pdone) {
    rc = launch_status(pkv::launch_prefill(out_prefill, q_prefill, cu_q_lens, k_cache, v_cache,
                                           nullptr, nullptr, block_tables_prefill,
                                           context_lens_prefill, B_prefill, total_q, max_q_len,
                                           Hq, Hkv, num_blocks, max_blocks_per_seq, scale, 0,
                                           pplan, prefill_workspace, s),
                       "pkv_attn_prefill_decode");
    if (rc) return rc;
  }
  if (!ddone)
    return launch_status(pkv::launch_decode(out_decode, q_decode, k_cache, v_cache,
                                            block_tables_decode, context_lens_decode, B_decode,
                                            Hq, Hkv, num_blocks, max_blocks_per_seq, scale, 0,
                                            dplan, decode_workspace, s),
                         "pkv_attn_prefill_decode");
  return PKV_OK;
}

int pkv_attn_prefill_decode_int8(
    void* out_prefill, const void* q_prefill, const int32_t* cu_q_lens,
    const int32_t* block_tables_prefill, const int32_t* context_lens_prefill, int32_t B_prefill,
    int32_t total_q, int32_t max_q_len, int32_t max_context_len_prefill, void* out_decode,
    const void* q_decode, const int32_t* block_tables_decode, const int32_t* context_lens_decode,
    int32_t B_decode, int32_t max_context_len_decode, const void* k_codes, const void* v_codes,
    const float* k_scales, const float* v_scales, int32_t Hq, int32_t Hkv, int32_t D,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
    void* prefill_workspace, size_t prefill_workspace_bytes, void* decode_workspace,
    size_t decode_workspace_bytes, void* stream) {
  if (((B_prefill > 0 && total_q > 0) || B_decode > 0) && (!k_scales || !v_scales))
    return fail(PKV_EINVAL, "null pointer argument");
  pkv::PrefillPlan pplan;
  bool pdone = true;
  int rc = check_prefill(out_prefill, q_prefill, cu_q_lens, k_codes, v_codes,
                         block_tables_prefill, context_lens_prefill, B_prefill, total_q,
                         max_q_len, Hq, Hkv, D, block_size, num_blocks, max_blocks_per_seq,
                         max_context_len_prefill, 0, scale, prefill_workspace,
                         prefill_workspace_bytes, stream, pplan, pdone);
  if (rc) return rc;
  pkv::DecodePlan dplan;
  bool ddone = false;
  rc = check_decode(out_decode, q_decode, k_codes, v_codes, block_tables_decode,
                    context_lens_decode, B_decode, Hq, Hkv, D, block_size, num_blocks,
                    max_blocks_per_seq, max_context_len_decode, scale, decode_workspace,
                    decode_workspace_bytes, stream, dplan, ddone);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!pdone && !ddone) {
    if (out_prefill == out_decode) return fail(PKV_EINVAL, "the two outputs must differ");
    if (pplan.ws_bytes && dplan.ws_bytes && prefill_workspace == decode_workspace)
      return fail(PKV_EINVAL, "the two workspaces must differ");
    if (pkv::mixed_plan_fits(dplan, Hq / Hkv))
      return launch_status(
          pkv::launch_prefill_decode_int8(
              out_prefill, q_prefill, cu_q_lens, block_tables_prefill, context_lens_prefill,
              B_prefill, total_q, max_q_len, pplan, prefill_workspace, out_decode, q_decode,
              block_tables_decode, context_lens_decode, B_decode, dplan, decode_workspace,
              k_codes, v_codes, k_scales, v_scales, Hq, Hkv, num_blocks, max_blocks_per_seq,
              scale, s),
          "pkv_attn_prefill_decode_int8");
  }
  // one half only, or a shape the one-grid launch does not take: the two
  // launches one after the other
  if (!pdone) {
    rc = launch_status(pkv::launch_prefill(out_prefill, q_prefill, cu_q_lens, k_codes, v_codes,
                                           k_scales, v_scales, block_tables_prefill,
                                           context_lens_prefill, B_prefill, total_q, max_q_len,
                                           Hq, Hkv, num_blocks, max_blocks_per_seq, scale, 0,
                                           pplan, prefill_workspace, s),
                       "pkv_attn_prefill_decode_int8");
    if (rc) return rc;
  }
  if (!ddone)
    return launch_status(pkv::launch_decode_int8(out_decode, q_decode, k_codes, v_codes,
                                                 k_scales, v_scales, block_tables_decode,
                                                 context_lens_decode, B_decode, Hq, Hkv,
                                                 num_blocks, max_blocks_per_seq, scale, dplan,
                                                 decode_workspace, s),
                         "pkv_attn_prefill_decode_int8");
  return PKV_OK;
}

int pkv_attn_prefill_decode_append(
    void* out_prefill, const void* q_prefill, const int32_t* cu_q_lens,
    const int32_t* block_tables_prefill, const int32_t* context_lens_prefill, int32_t B_prefill,
    int32_t total_q, int32_t max_q_len, int32_t max_context_len_prefill, void* out_decode,
    const void* q_decode, const int32_t* block_tables_decode, const int32_t* context_lens_decode,
    int32_t B_decode, int32_t max_context_len_decode, const void* k_new, const void* v_new,
    const int32_t* slot_mapping, void* k_cache, void* v_cache, int32_t Hq, int32_t Hkv, int32_t D,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
    void* prefill_workspace, size_t prefill_workspace_bytes, void* decode_workspace,
    size_t decode_workspace_bytes, void* stream) {
  pkv::PrefillPlan pplan;
  bool pdone = true;
  int rc = check_prefill(out_prefill, q_prefill, cu_q_lens, k_cache, v_cache,
                         block_tables_prefill, context_lens_prefill, B_prefill, total_q,
                         max_q_len, Hq, Hkv, D, block_size, num_blocks, max_blocks_per_seq,
                         max_context_len_prefill, 0, scale, prefill_workspace,
                         prefill_workspace_bytes, stream, pplan, pdone);
  if (rc) return rc;
  pkv::DecodePlan dplan;
  bool ddone = false;
  rc = check_decode(out_decode, q_decode, k_cache, v_cache, block_tables_decode,
                    context_lens_decode, B_decode, Hq, Hkv, D, block_size, num_blocks,
                    max_blocks_per_seq, max_context_len_decode, scale, decode_workspace,
                    decode_workspace_bytes, stream, dplan, ddone);
  if (rc) return rc;
  if (pdone && ddone) return PKV_OK;
  const int32_t n_chunk = pdone ? 0 : total_q;            // chunk rows, then decode rows
  const int32_t n_rows = n_chunk + (ddone ? 0 : B_decode);
  if (!k_new || !v_new || !slot_mapping) return fail(PKV_EINVAL, "null pointer argument");
  if (k_cache == v_cache) return fail(PKV_EINVAL, "k_cache and v_cache must differ");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_mode()) {
    rc = validate_slots(slot_mapping, n_rows, num_blocks, s);
    if (rc) return rc;
  }
  if (!pdone && !ddone) {
    if (out_prefill == out_decode) return fail(PKV_EINVAL, "the two outputs must differ");
    if (pplan.ws_bytes && dplan.ws_bytes && prefill_workspace == decode_workspace)
      return fail(PKV_EINVAL, "the two workspaces must differ");
    if (pkv::mixed_plan_fits(dplan, Hq / Hkv))
      return launch_status(
          pkv::launch_prefill_decode_append(
              out_prefill, q_prefill, cu_q_lens, block_tables_prefill, context_lens_prefill,
              B_prefill, total_q, max_q_len, pplan, prefill_workspace, out_decode, q_decode,
              block_tables_decode, context_lens_decode, B_decode, dplan, decode_workspace, k_new,
              v_new, slot_mapping, k_cache, v_cache, Hq, Hkv, num_blocks, max_blocks_per_seq,
              scale, s),
          "pkv_attn_prefill_decode_append");
  }
  // one half only, or a shape the one-grid launch does not take: the append,
  // then the attention launches one after the other
  rc = launch_status(pkv::launch_append(k_new, v_new, slot_mapping, k_cache, v_cache, n_rows,
                                        num_blocks, Hkv, D, s),
                     "pkv_attn_prefill_decode_append");
  if (rc) return rc;
  if (!pdone) {
    rc = launch_status(pkv::launch_prefill(out_prefill, q_prefill, cu_q_lens, k_cache, v_cache,
                                           nullptr, nullptr, block_tables_prefill,
                                           context_lens_prefill, B_prefill, total_q, max_q_len,
                                           Hq, Hkv, num_blocks, max_blocks_per_seq, scale, 0,
                                           pplan, prefill_workspace, s),
                       "pkv_attn_prefill_decode_append");
    if (rc) return rc;
  }
  if (!ddone)
    return launch_status(pkv::launch_decode(out_decode, q_decode, k_cache, v_cache,
                                            block_tables_decode, context_lens_decode, B_decode,
                                            Hq, Hkv, num_blocks, max_blocks_per_seq, scale, 0,
                                            dplan, decode_workspace, s),
                         "pkv_attn_prefill_decode_append");
  return PKV_OK;
}

}  // extern "C"
