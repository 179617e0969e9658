// One launch for the attention of a mixed step: the chunked-prefill
// workgroups of the step's prefill sequences and the decode workgroups of its
// decode sequences in one grid.
//
// What is computed (Module 12 page, "Why chunked prefill": a scheduler step
// carries one token for each decoding sequence beside prompt chunks, and
// every layer runs attention for all of them over the pages): exactly what
// the chunked-prefill call and the decode call compute for their halves of
// the step, with the same per-workgroup arithmetic.
//
// Why one launch.  At the sizes of such a step neither half fills the chip
// on its own for long: a 512-query chunk of a small model is a few hundred
// workgroups each bounded by a chain of memory round trips, and a handful of
// decode sequences even less.  Two launches run one after the other (a HIP
// graph executes a layer's kernels in order on one queue), so the step paid
// the sum of two latency-bound kernels per layer.  In one grid the decode
// workgroups fill the compute-unit slots the chunk leaves free and both
// halves' latencies overlap.  Both kinds are 4 waves (the chunk's four
// 32-row waves; decode with one KV head and four page-part waves per
// workgroup, its split plan unchanged), with the chunk kernel's register
// budget (two workgroups per CU) and the LDS of both bodies.  Chunk
// workgroups come first in the grid (they are the longer ones); both halves
// keep their own KV-head-fastest order, so each KV head's workgroups share
// an XCD as in the separate launches.
// Every decode workgroup here has four waves: the int8 page staging buffers
// are sized for that, which leaves room in the LDS for the int8 chunk body.
#define PKV_I8_LDS_WAVES 4
#include "decode_kernel.h"
#include "prefill_kernel.h"
#include <algorithm>

namespace pkv {

namespace {

template <int G, int U>
__global__ void __launch_bounds__(pf::kWaves * kWave, 2)
mixed_kernel(const pf::PrefillArgs pa, const dec::DecodeArgs da, const int n_prefill_wgs) {
  const int bid = blockIdx.x;
  if (bid < n_prefill_wgs)
    pf::prefill_body<false>(pa, bid);
  else
    dec::decode_body<dec::Bf16Page, G, U, pf::kWaves, false>(da, bid - n_prefill_wgs);
}

template <int G, int U>
hipError_t launch_g(const pf::PrefillArgs& pa, const dec::DecodeArgs& da, int n_pre, int n_dec,
                    hipStream_t stream) {
  hipLaunchKernelGGL((mixed_kernel<G, U>), dim3(n_pre + n_dec), dim3(pf::kWaves * kWave), 0,
                     stream, pa, da, n_pre);
  return hipGetLastError();
}

// The same over int8 pages: the int8 chunk body (its code ring fills most of
// the LDS, one workgroup per CU) beside the int8 decode body with one KV
// head and four page-part waves per workgroup.
template <int G, int U>
__global__ void __launch_bounds__(pf::kWaves * kWave, 1)
mixed_int8_kernel(const pf::PrefillArgs pa, const dec::DecodeArgs da, const int n_prefill_wgs) {
  static_assert(pf::kWaves <= dec::kI8LdsWaves, "int8 staging buffers for every wave");
  const int bid = blockIdx.x;
  if (bid < n_prefill_wgs)
    pf::prefill_body<true>(pa, bid);
  else
    dec::decode_body<dec::Int8Page, G, U, pf::kWaves, false>(da, bid - n_prefill_wgs);
}

template <int G, int U>
hipError_t launch_int8_g(const pf::PrefillArgs& pa, const dec::DecodeArgs& da, int n_pre,
                         int n_dec, hipStream_t stream) {
  hipLaunchKernelGGL((mixed_int8_kernel<G, U>), dim3(n_pre + n_dec), dim3(pf::kWaves * kWave), 0,
                     stream, pa, da, n_pre);
  return hipGetLastError();
}

// The same step with its append in the grid too (Module 12 page, model.py
// forward: each layer writes the step's K/V into the cache and attends over
// the cached prefix plus those rows).  Nothing in the grid reads a slot that
// the grid writes: the chunk workgroups read their chunk's own rows from
// k_new (pa.k_new), the decode workgroups take their sequence's new row from
// k_new and write it into its slot (the fused decode-append body), and the
// last n_app workgroups copy the chunk rows into their slots.
struct AppendArgs {
  const u32x4* k_new;
  const u32x4* v_new;
  const int32_t* slots;          // the chunk rows' slots (first total_q entries of the step's)
  u32x4* k_cache;
  u32x4* v_cache;
  int64_t n_items;               // total_q * 2 * Hkv * chunks_per_head
  int Hkv, chunks_per_head;
  int64_t num_slots;
};

template <int G, int U>
__global__ void __launch_bounds__(pf::kWaves * kWave, 2)
mixed_append_kernel(const pf::PrefillArgs pa, const dec::DecodeArgs da, const AppendArgs ap,
                    const int n_prefill_wgs, const int n_decode_wgs) {
  const int bid = blockIdx.x;
  if (bid < n_prefill_wgs) {
    pf::prefill_body<false, true>(pa, bid);
  } else if (bid < n_prefill_wgs + n_decode_wgs) {
    dec::decode_body<dec::Bf16Page, G, U, pf::kWaves, true>(da, bid - n_prefill_wgs);
  } else {
    const int64_t nt = (int64_t)(gridDim.x - n_prefill_wgs - n_decode_wgs) * blockDim.x;
    append_rows(ap.k_new, ap.v_new, ap.slots, ap.k_cache, ap.v_cache, ap.n_items, ap.Hkv,
                ap.chunks_per_head, ap.num_slots,
                (int64_t)(bid - n_prefill_wgs - n_decode_wgs) * blockDim.x + threadIdx.x, nt);
  }
}

template <int G, int U>
hipError_t launch_append_g(const pf::PrefillArgs& pa, const dec::DecodeArgs& da,
                           const AppendArgs& ap, int n_pre, int n_dec, int n_app,
                           hipStream_t stream) {
  hipLaunchKernelGGL((mixed_append_kernel<G, U>), dim3(n_pre + n_dec + n_app),
                     dim3(pf::kWaves * kWave), 0, stream, pa, da, ap, n_pre, n_dec);
  return hipGetLastError();
}

}  // namespace

// Group sizes up to 4: at 8 the decode body's LDS (its page-part exchange
// grows with the group) and the chunk's would not leave room for two
// workgroups per CU.
bool mixed_plan_fits(const DecodePlan& dplan, int G) {
  return dplan.parts == pf::kWaves && (G == 1 || G == 2 || G == 4);
}

hipError_t launch_prefill_decode(void* out_p, const void* q_p, const int32_t* cu_q,
                                 const int32_t* bt_p, const int32_t* ctx_p, int B_p, int total_q,
                                 int max_q_len, const PrefillPlan& pplan, void* ws_p,
                                 void* out_d, const void* q_d, const int32_t* bt_d,
                                 const int32_t* ctx_d, int B_d, const DecodePlan& dplan,
                                 void* ws_d, const void* k_cache, const void* v_cache, int Hq,
                                 int Hkv, int num_blocks, int max_blocks, float scale,
                                 hipStream_t stream) {
  if (!mixed_plan_fits(dplan, Hq / Hkv)) return hipErrorInvalidValue;
  const pf::PrefillArgs pa =
      pf::make_prefill_args(out_p, q_p, cu_q, k_cache, v_cache, nullptr, nullptr, bt_p, ctx_p,
                            B_p, total_q, max_q_len, Hq, Hkv, num_blocks, max_blocks, scale, 0,
                            pplan, ws_p);
  // One KV head per decode workgroup (four page-part waves); the splits,
  // their page ranges and the workspace layout are those of the plan.
  DecodePlan dp = dplan;
  dp.heads_per_wg = 1;
  const dec::DecodeArgs da =
      dec::make_args(out_d, q_d, k_cache, v_cache, nullptr, nullptr, bt_d, ctx_d, B_d, Hq, Hkv,
                     num_blocks, max_blocks, scale, dp, dec::workspace_buffers(dp, ws_d), 0);
  const int64_t n_pre = (int64_t)B_p * pa.qtiles * pa.splits * Hkv;
  const int64_t n_dec = (int64_t)B_d * dp.splits * Hkv;
  if (n_pre + n_dec > 0x7fffffff) return hipErrorInvalidValue;
  switch (Hq / Hkv) {
    case 1: return launch_g<1, PKV_DECODE_U_G1>(pa, da, (int)n_pre, (int)n_dec, stream);
    case 2: return launch_g<2, PKV_DECODE_U_G2>(pa, da, (int)n_pre, (int)n_dec, stream);
    case 4: return launch_g<4, PKV_DECODE_U_G4>(pa, da, (int)n_pre, (int)n_dec, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_decode_int8(void* out_p, const void* q_p, const int32_t* cu_q,
                                      const int32_t* bt_p, const int32_t* ctx_p, int B_p,
                                      int total_q, int max_q_len, const PrefillPlan& pplan,
                                      void* ws_p, void* out_d, const void* q_d,
                                      const int32_t* bt_d, const int32_t* ctx_d, int B_d,
                                      const DecodePlan& dplan, void* ws_d, const void* k_codes,
                                      const void* v_codes, const float* k_scales,
                                      const float* v_scales, int Hq, int Hkv, int num_blocks,
                                      int max_blocks, float scale, hipStream_t stream) {
  if (!mixed_plan_fits(dplan, Hq / Hkv)) return hipErrorInvalidValue;
  const pf::PrefillArgs pa =
      pf::make_prefill_args(out_p, q_p, cu_q, k_codes, v_codes, k_scales, v_scales, bt_p, ctx_p,
                            B_p, total_q, max_q_len, Hq, Hkv, num_blocks, max_blocks, scale, 0,
                            pplan, ws_p);
  DecodePlan dp = dplan;
  dp.heads_per_wg = 1;
  const dec::DecodeArgs da =
      dec::make_args(out_d, q_d, k_codes, v_codes, k_scales, v_scales, bt_d, ctx_d, B_d, Hq, Hkv,
                     num_blocks, max_blocks, scale, dp, dec::workspace_buffers(dp, ws_d), 0);
  const int64_t n_pre = (int64_t)B_p * pa.qtiles * pa.splits * Hkv;
  const int64_t n_dec = (int64_t)B_d * dp.splits * Hkv;
  if (n_pre + n_dec > 0x7fffffff) return hipErrorInvalidValue;
  switch (Hq / Hkv) {
    case 1: return launch_int8_g<1, PKV_DECODE_I8_U_G1>(pa, da, (int)n_pre, (int)n_dec, stream);
    case 2: return launch_int8_g<2, PKV_DECODE_I8_U_G2>(pa, da, (int)n_pre, (int)n_dec, stream);
    case 4: return launch_int8_g<4, PKV_DECODE_I8_U_G4>(pa, da, (int)n_pre, (int)n_dec, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_decode_append(
    void* out_p, const void* q_p, const int32_t* cu_q, const int32_t* bt_p, const int32_t* ctx_p,
    int B_p, int total_q, int max_q_len, const PrefillPlan& pplan, void* ws_p, void* out_d,
    const void* q_d, const int32_t* bt_d, const int32_t* ctx_d, int B_d, const DecodePlan& dplan,
    void* ws_d, const void* k_new, const void* v_new, const int32_t* slot_mapping,
    void* k_cache, void* v_cache, int Hq, int Hkv, int num_blocks, int max_blocks, float scale,
    hipStream_t stream) {
  if (!mixed_plan_fits(dplan, Hq / Hkv)) return hipErrorInvalidValue;
  pf::PrefillArgs pa =
      pf::make_prefill_args(out_p, q_p, cu_q, k_cache, v_cache, nullptr, nullptr, bt_p, ctx_p,
                            B_p, total_q, max_q_len, Hq, Hkv, num_blocks, max_blocks, scale, 0,
                            pplan, ws_p);
  pa.k_new = static_cast<const u32x4*>(k_new);
  pa.v_new = static_cast<const u32x4*>(v_new);
  DecodePlan dp = dplan;
  dp.heads_per_wg = 1;
  dec::DecodeArgs da =
      dec::make_args(out_d, q_d, k_cache, v_cache, nullptr, nullptr, bt_d, ctx_d, B_d, Hq, Hkv,
                     num_blocks, max_blocks, scale, dp, dec::workspace_buffers(dp, ws_d), 0);
  // decode sequence b's new row is row total_q + b of k_new / v_new
  const int64_t row_chunks = (int64_t)Hkv * (kD * 2 / 16);
  da.k_new = static_cast<const u32x4*>(k_new) + total_q * row_chunks;
  da.v_new = static_cast<const u32x4*>(v_new) + total_q * row_chunks;
  da.k_pool = static_cast<u32x4*>(k_cache);
  da.v_pool = static_cast<u32x4*>(v_cache);
  AppendArgs ap;
  ap.k_new = static_cast<const u32x4*>(k_new);
  ap.v_new = static_cast<const u32x4*>(v_new);
  ap.slots = slot_mapping;
  ap.k_cache = static_cast<u32x4*>(k_cache);
  ap.v_cache = static_cast<u32x4*>(v_cache);
  ap.chunks_per_head = kD * 2 / 16;
  ap.Hkv = Hkv;
  ap.n_items = (int64_t)total_q * 2 * row_chunks;
  ap.num_slots = (int64_t)num_blocks * kPage;
  const int64_t n_pre = (int64_t)B_p * pa.qtiles * pa.splits * Hkv;
  const int64_t n_dec = (int64_t)B_d * dp.splits * Hkv;
  // one 16-byte item per thread and round; at most 64 workgroups
  const int64_t n_app = std::min<int64_t>(64, (ap.n_items + 255) / 256);
  if (n_pre + n_dec + n_app > 0x7fffffff) return hipErrorInvalidValue;
  switch (Hq / Hkv) {
    case 1: return launch_append_g<1, PKV_DECODE_U_G1>(pa, da, ap, (int)n_pre, (int)n_dec, (int)n_app, stream);
    case 2: return launch_append_g<2, PKV_DECODE_U_G2>(pa, da, ap, (int)n_pre, (int)n_dec, (int)n_app, stream);
    case 4: return launch_append_g<4, PKV_DECODE_U_G4>(pa, da, ap, (int)n_pre, (int)n_dec, (int)n_app, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
