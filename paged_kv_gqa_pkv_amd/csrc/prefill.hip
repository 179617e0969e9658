// Chunked-prefill key-split planner and launcher; the kernel is in
// prefill_kernel.h.
#include "prefill_kernel.h"

namespace pkv {

using namespace pf;

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// Key-split planner.  Row tiles x KV heads x sequences give the "groups";
// each group's key range is cut into splits of tiles_per_split 64-key tiles.
// The grid runs in rounds of num_cus * PKV_PREFILL_WG_PER_CU workgroups (1:
// counting the two bf16 workgroups a CU holds measured slower); for
// every split count the planner estimates rounds * (tiles per split + a fixed
// workgroup cost) plus a merge cost when the key range is split, and keeps
// the cheapest (fewest splits on ties).  Host-known bounds only.
PrefillPlan plan_prefill(int B, int max_q_len, int Hq, int Hkv, int max_context_len,
                         int num_cus) {
  PrefillPlan p{};
  const int G = Hq / Hkv;
  p.qtiles = max(1, (max_q_len * G + kRowsPerWG - 1) / kRowsPerWG);
  const int64_t groups = (int64_t)B * p.qtiles * Hkv;
  const int max_tiles = max(1, (max_context_len + kTileKeys - 1) / kTileKeys);
  const int64_t slots = (int64_t)PKV_PREFILL_WG_PER_CU * max(1, num_cus);
  int best_s = 0, best_tps = 0;
  int64_t best_cost = -1;
  int last_tps = -1;
  for (int s_try = 1; s_try <= kMaxSplits; ++s_try) {
    int tps = (max_tiles + s_try - 1) / s_try;
    if (tps > kMaxTilesPerSplit) continue;
    if (tps < PKV_PREFILL_MIN_TILES && s_try > 1) break;
    if (tps == last_tps) continue;
    last_tps = tps;
    const int splits = (max_tiles + tps - 1) / tps;
    const int64_t rounds = (groups * splits + slots - 1) / slots;
    const int64_t cost = rounds * (tps + PKV_PREFILL_WG_COST_TILES) +
                         (splits > 1 ? PKV_PREFILL_MERGE_COST_TILES : 0);
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best_s = splits; best_tps = tps; }
  }
  p.ok = best_s > 0;                       // contexts up to 32 * 64 * 64 = 131072 keys
  p.splits = best_s > 0 ? best_s : 1;
  p.tiles_per_split = best_s > 0 ? best_tps : max_tiles;
  if (p.ok && p.splits > 1) {
    p.ws_acc_bytes = align256((size_t)groups * p.splits * kRowsPerWG * kD * sizeof(float));
    p.ws_ml_bytes = align256((size_t)groups * p.splits * kRowsPerWG * 2 * sizeof(float));
    p.ws_counter_bytes = align256((size_t)groups * sizeof(int));
  }
  p.ws_bytes = p.ws_acc_bytes + p.ws_ml_bytes + p.ws_counter_bytes;
  return p;
}

hipError_t launch_prefill(void* out, const void* q, const int32_t* cu_q, const void* k_cache,
                          const void* v_cache, const float* k_scales, const float* v_scales,
                          const int32_t* block_tables,
                          const int32_t* ctx_lens, int B, int total_q, int max_q_len, int Hq,
                          int Hkv, int num_blocks, int max_blocks, float scale, int window,
                          const PrefillPlan& plan, void* workspace, hipStream_t stream) {
  if (B == 0 || total_q == 0 || max_q_len == 0) return hipSuccess;
  const PrefillArgs a = make_prefill_args(out, q, cu_q, k_cache, v_cache, k_scales, v_scales,
                                          block_tables, ctx_lens, B, total_q, max_q_len, Hq, Hkv,
                                          num_blocks, max_blocks, scale, window, plan, workspace);
  const unsigned grid = (unsigned)((int64_t)B * a.qtiles * a.splits * Hkv);
  if (k_scales)
    hipLaunchKernelGGL(prefill_kernel<true>, dim3(grid), dim3(kWaves * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_kernel<false>, dim3(grid), dim3(kWaves * kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
