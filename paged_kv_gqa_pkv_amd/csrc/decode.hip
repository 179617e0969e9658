// Decode launchers, split planner and the per-GPU scratch array of the
// decode call that allocates nothing; the kernel is in decode_kernel.h.
#include "decode_kernel.h"

#include <mutex>
#include <vector>

namespace pkv {

using namespace dec;

namespace {

template <class P, int G, int U, bool kAppend = false>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  constexpr int kMaxWaves = max_waves_for(G);
  const int waves = a.heads_per_wg * a.parts;
  if (a.heads_per_wg < 1 || a.parts < 1 || waves > kMaxWaves || a.Hkv % a.heads_per_wg ||
      a.pages_per_split % a.parts || a.pages_per_split / a.parts > kMaxPagesPerWave)
    return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((int64_t)a.B * a.splits * (a.Hkv / a.heads_per_wg));
  hipLaunchKernelGGL((decode_kernel<P, G, U, kMaxWaves, kAppend>), dim3(grid),
                     dim3(waves * kWave), 0, stream, a);
  return hipGetLastError();
}


// One group size: bf16 pages from PKV_DECODE_MFMA_MIN_G on run the matrix-core
// policy; the pages per pipeline stage U follow each policy's register budget.
template <class P, int G, int U, int UI8, bool kAppend>
hipError_t launch_policy(const DecodeArgs& a, hipStream_t stream) {
  if constexpr (std::is_same<P, Int8Page>::value)
    return launch_g<Int8Page, G, UI8, kAppend>(a, stream);
  else if constexpr (G >= PKV_DECODE_MFMA_MIN_G)
    return launch_g<Bf16MfmaPage, G, PKV_DECODE_B16M_U, kAppend>(a, stream);
  else
    return launch_g<P, G, U, kAppend>(a, stream);
}

// Instantiations by group size G = Hq / Hkv.
template <class P, bool kAppend = false>
hipError_t launch_by_group(const DecodeArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_policy<P, 1, PKV_DECODE_U_G1, PKV_DECODE_I8_U_G1, kAppend>(a, stream);
    case 2: return launch_policy<P, 2, PKV_DECODE_U_G2, PKV_DECODE_I8_U_G2, kAppend>(a, stream);
    case 4: return launch_policy<P, 4, PKV_DECODE_U_G4, PKV_DECODE_I8_U_G4, kAppend>(a, stream);
    case 8: return launch_policy<P, 8, PKV_DECODE_U_G8, PKV_DECODE_I8_U_G8, kAppend>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

// Library-owned split buffers for callers that cannot allocate
// (launch_decode_noalloc).  One array per device, held until the process
// ends: the arrival counters first (a fixed region, so that every call finds
// them at the same place and at zero: each call leaves the counters it used
// at zero, and the region is cleared once per device before the first use),
// then the (m, l) and acc partials of the call in flight, which need no
// initialisation.  Host code never passes `scratch` itself to a kernel (its
// name is a host-side stand-in there): it uses the device address obtained
// from hipGetSymbolAddress, kept per device.
static __device__ __align__(256) char scratch[PKV_NOALLOC_SCRATCH_BYTES];
constexpr size_t kScratchCounterBytes = PKV_NOALLOC_COUNTER_BYTES;
static_assert(kScratchCounterBytes % 256 == 0 && kScratchCounterBytes < PKV_NOALLOC_SCRATCH_BYTES,
              "counter region inside the scratch array");

__global__ void __launch_bounds__(256) zero_words_kernel(int* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// Device address of `scratch` on the current device; on the first call for a
// device the symbol is resolved (with that device current) and its counter
// region cleared by a fill kernel on `stream` (a kernel, not a memset, so
// that the clear is also valid inside a captured graph).
hipError_t scratch_address(char** out, hipStream_t stream) {
  static std::mutex mu;
  static std::vector<char*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    const int words = (int)(kScratchCounterBytes / sizeof(int));
    hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                       static_cast<int*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<char*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// Split planner.  A workgroup streams one split of one (sequence, head
// group): heads_per_wg KV heads times `parts` waves per head, each wave over
// pages_per_split / parts pages.  A compute unit holds max_waves_for(G)
// waves (times PKV_DECODE_WG_PER_CU / 2, the register budget's two waves per
// SIMD being the default), so the grid runs in "rounds" of num_cus times
// the workgroups that fit.  For each split length the planner estimates the
// time as rounds * (pages per wave + a fixed per-workgroup cost) plus, when
// the context is split, a merge cost that grows with the number of splits
// (their arrivals on one counter are serialised), and keeps the cheapest
// (fewest splits on ties).  Pages per wave are PKV_DECODE_MIN_PPW .. 64 (one
// VGPR of page ids).  Only host-known sizes enter, so no device->host sync is
// needed.
DecodePlan plan_decode(int B, int Hq, int Hkv, int max_context_len, int num_cus) {
  DecodePlan p{};
  const int G = max(1, Hq / max(1, Hkv));
  const int max_waves = max_waves_for(G);
  int hg = 1;                                 // largest divisor of Hkv within the caps
  for (int d = 1; d <= min(max_waves, PKV_DECODE_MAX_HG); ++d)
    if (Hkv % d == 0) hg = d;
  const int pw = max(1, min(PKV_DECODE_PARTS, max_waves / hg));
  p.heads_per_wg = hg;
  p.parts = pw;
  const int max_pages = max(1, (max_context_len + kPage - 1) / kPage);
  const int64_t units = max(1, B * (Hkv / hg));
  const int wg_per_cu = max(1, max_waves * PKV_DECODE_WG_PER_CU / 2 / (hg * pw));
  const int64_t slots = (int64_t)wg_per_cu * max(1, num_cus);
  int best_s = 1, best_ppw = 0;
  int64_t best_cost = -1;
  int last_ppw = -1;
  // the G <= 2 kernels reduce pages in pairs: an odd count leaves one alone
  const int ustep = G <= 2 ? 2 : 1;
  for (int s_try = 1; s_try <= max_pages; ++s_try) {
    int ppw = (max_pages + s_try * pw - 1) / (s_try * pw);
    ppw = (ppw + ustep - 1) / ustep * ustep;
    if (ppw > kMaxPagesPerWave) continue;
    if (ppw < PKV_DECODE_MIN_PPW) ppw = PKV_DECODE_MIN_PPW;
    if (ppw == last_ppw) continue;
    last_ppw = ppw;
    const int splits = (max_pages + ppw * pw - 1) / (ppw * pw);
    const int64_t rounds = (units * splits + slots - 1) / slots;
    // in eighths of a page-time
    const int64_t cost = rounds * (ppw + PKV_DECODE_WG_COST_PAGES) * 8 +
                         (splits > 1 ? PKV_DECODE_MERGE_COST_PAGES * 8 +
                                           (int64_t)splits * PKV_DECODE_SPLIT_COST_EIGHTHS
                                     : 0);
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best_s = splits; best_ppw = ppw; }
    if (ppw == PKV_DECODE_MIN_PPW) break;
  }
#if PKV_DECODE_FORCE_PPW > 0
  // tuning builds only: a fixed number of pages per wave
  best_ppw = min(PKV_DECODE_FORCE_PPW, kMaxPagesPerWave);
  best_s = (max_pages + best_ppw * pw - 1) / (best_ppw * pw);
#endif
  // Long page loops (bandwidth-bound) run faster with two KV heads per
  // workgroup, whose waves then read two heads' rows of the same pages
  // together; short ones (latency-bound) spread better over the compute
  // units with one.  The split length stays as planned.
  if (PKV_DECODE_WIDE_PPW > 0 && best_ppw >= PKV_DECODE_WIDE_PPW && hg == 1 && Hkv % 2 == 0 &&
      2 * pw <= max_waves) {
    hg = 2;
    p.heads_per_wg = hg;
  }
  p.splits = best_s;
  p.pages_per_split = best_ppw * pw;
  if (best_s > 1) {
    p.ws_ml_bytes = align256((size_t)B * Hq * best_s * 2 * sizeof(float));
    p.ws_acc_bytes = align256((size_t)B * Hq * best_s * kD * sizeof(float));
    // one counter per (sequence, KV head) whatever the heads per workgroup,
    // so that a launch with one head per workgroup fits the same workspace
    p.ws_counter_bytes = align256((size_t)B * Hkv * sizeof(int));
  }
  p.ws_bytes = p.ws_ml_bytes + p.ws_acc_bytes + p.ws_counter_bytes;
  return p;
}

hipError_t launch_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* ctx_lens, int B, int Hq,
                         int Hkv, int num_blocks, int max_blocks, float scale, int window,
                         const DecodePlan& plan, void* workspace, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const DecodeArgs a = make_args(out, q, k_cache, v_cache, nullptr, nullptr, block_tables,
                                 ctx_lens, B, Hq, Hkv, num_blocks, max_blocks, scale, plan,
                                 workspace_buffers(plan, workspace), window);
  return launch_by_group<Bf16Page>(a, Hq / Hkv, stream);
}

hipError_t launch_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, const int32_t* block_tables,
                                const int32_t* ctx_lens, int B, int Hq, int Hkv, int num_blocks,
                                int max_blocks, float scale, const DecodePlan& plan,
                                void* workspace, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  DecodeArgs a = make_args(out, q, k_cache, v_cache, nullptr, nullptr, block_tables, ctx_lens, B,
                           Hq, Hkv, num_blocks, max_blocks, scale, plan,
                           workspace_buffers(plan, workspace), 0);
  a.k_new = static_cast<const u32x4*>(k_new);
  a.v_new = static_cast<const u32x4*>(v_new);
  a.k_pool = static_cast<u32x4*>(k_cache);
  a.v_pool = static_cast<u32x4*>(v_cache);
  return launch_by_group<Bf16Page, true>(a, Hq / Hkv, stream);
}

bool noalloc_fits(const DecodePlan& plan, int B, int Hkv) {
  if (plan.splits <= 1) return true;
  return plan.ws_counter_bytes <= kScratchCounterBytes &&
         plan.ws_ml_bytes + plan.ws_acc_bytes <= PKV_NOALLOC_SCRATCH_BYTES - kScratchCounterBytes;
}

hipError_t launch_decode_noalloc(void* out, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* ctx_lens, int B, int Hq, int Hkv, int num_blocks,
                                 int max_blocks, float scale, const DecodePlan& plan,
                                 hipStream_t stream) {
  if (B == 0) return hipSuccess;
  if (!noalloc_fits(plan, B, Hkv)) return hipErrorInvalidValue;
  char* base = nullptr;
  const hipError_t e = scratch_address(&base, stream);
  if (e != hipSuccess) return e;
  const SplitBuffers wsb{reinterpret_cast<float*>(base + kScratchCounterBytes),
                         reinterpret_cast<float*>(base + kScratchCounterBytes + plan.ws_ml_bytes),
                         reinterpret_cast<int*>(base)};
  const DecodeArgs a = make_args(out, q, k_cache, v_cache, nullptr, nullptr, block_tables,
                                 ctx_lens, B, Hq, Hkv, num_blocks, max_blocks, scale, plan, wsb,
                                 0);
  return launch_by_group<Bf16Page>(a, Hq / Hkv, stream);
}

hipError_t launch_decode_append_int8(void* out, const void* q, const void* k_new,
                                     const void* v_new, void* k_codes, void* v_codes,
                                     float* k_scales, float* v_scales,
                                     const int32_t* block_tables, const int32_t* ctx_lens, int B,
                                     int Hq, int Hkv, int num_blocks, int max_blocks, float scale,
                                     const DecodePlan& plan, void* workspace,
                                     hipStream_t stream) {
  if (B == 0) return hipSuccess;
  DecodeArgs a = make_args(out, q, k_codes, v_codes, k_scales, v_scales, block_tables, ctx_lens,
                           B, Hq, Hkv, num_blocks, max_blocks, scale, plan,
                           workspace_buffers(plan, workspace), 0);
  a.k_new = static_cast<const u32x4*>(k_new);
  a.v_new = static_cast<const u32x4*>(v_new);
  a.k_pool = static_cast<u32x4*>(k_codes);
  a.v_pool = static_cast<u32x4*>(v_codes);
  a.ks_pool = k_scales;
  a.vs_pool = v_scales;
  return launch_by_group<Int8Page, true>(a, Hq / Hkv, stream);
}

hipError_t launch_decode_int8(void* out, const void* q, const void* k_codes, const void* v_codes,
                              const float* k_scales, const float* v_scales,
                              const int32_t* block_tables, const int32_t* ctx_lens, int B, int Hq,
                              int Hkv, int num_blocks, int max_blocks, float scale,
                              const DecodePlan& plan, void* workspace, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const DecodeArgs a = make_args(out, q, k_codes, v_codes, k_scales, v_scales, block_tables,
                                 ctx_lens, B, Hq, Hkv, num_blocks, max_blocks, scale, plan,
                                 workspace_buffers(plan, workspace), 0);
  return launch_by_group<Int8Page>(a, Hq / Hkv, stream);
}

}  // namespace pkv
