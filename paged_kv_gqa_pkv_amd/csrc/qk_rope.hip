// The step before attention, fused: per-head q/k RMSNorm, RoPE at each
// token's absolute position, and the write of the rotated k (and of v) into
// its page slot.
//
// What is computed (Module 12 page, model.py): rms_norm(x, w, eps) takes the
// mean of x^2 and its rsqrt in float32, casts x * inv back to bf16 and
// multiplies by the bf16 weight; apply_rope computes q * cos[pos] +
// rotate_half(q) * sin[pos] on bf16 tensors with rotate_half(x) =
// (-x[D/2:], x[:D/2]) and the cos/sin tables (both halves duplicated) given
// by the caller; forward does this for q and k of every new token, then
// writes k and v into the cache at the token's slot.  Every bf16 tensor
// operation of the listing rounds its result to bf16 here too (products of
// two bf16 values and sums of two of them are exact in float32 before that
// rounding), so the only difference from the listing's arithmetic is the
// order of the 128-term sum of squares.
//
// Layout of the work: one workgroup per token; 16 lanes own one row (head)
// of 128 values, 8 per lane (one 16-byte load), and the 16 row slots of the
// workgroup walk the token's Hq + 2 Hkv rows.  The sum of squares is a DPP
// reduction inside the 16-lane row; the rotate-half partner of dims
// 8s..8s+7 (dims +-64) sits in lane s ^ 8 of the same row, one DPP row
// rotation away.  The token's position and slot are found once per
// workgroup, as the slot-mapping kernel finds them (binary search over
// cu_new_lens), so no separate slot-mapping launch is needed.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

__device__ __forceinline__ float sum16(float x) {
  x += dpp_f<kDppQuadSwap1>(x);
  x += dpp_f<kDppQuadSwap2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  return x + dpp_f<kDppRowRor8>(x);
}

// float -> nearest bf16 (ties to even) -> float: the hardware convert
// (v_cvt_pk_bf16_f32) and a shift back.
__device__ __forceinline__ float round_bf16(float x) { return (float)(__bf16)x; }

struct QkRopeArgs {
  uint16_t* q_out;             // bf16 [T][Hq][D]
  const u32x4* q_in;           // bf16 [T][Hq][D]
  const u32x4* k_in;           // bf16 [T][Hkv][D]
  const u32x4* v_in;
  const u32x4* q_w;            // bf16 [D]
  const u32x4* k_w;
  const u32x4* cos_t;          // bf16 [max_pos][D]
  const u32x4* sin_t;
  const int32_t* block_tables; // [B][max_blocks]
  const int32_t* cu_new;       // [B+1]
  const int32_t* ctx_lens;     // [B]
  int32_t* slots;              // [T] out (may be null)
  u32x4* k_cache;              // bf16 [num_blocks][16][Hkv][D]
  u32x4* v_cache;
  int B, max_blocks, T, num_blocks, Hq, Hkv, max_pos;
  float eps;
};

__global__ void __launch_bounds__(256) qk_norm_rope_append_kernel(const QkRopeArgs a) {
  const int sub = threadIdx.x & 15;
  const int per_tok = a.Hq + 2 * a.Hkv;
  const int t = blockIdx.x;                  // one token per workgroup
  int lo = 0, hi = a.B;                      // sequence b with cu[b] <= t < cu[b+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_new[mid] <= t) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int p = a.ctx_lens[b] - (a.cu_new[b + 1] - a.cu_new[b]) + (t - a.cu_new[b]);
  int64_t slot = -1;
  if (p >= 0 && (p >> 4) < a.max_blocks) {
    const int blk = a.block_tables[(int64_t)b * a.max_blocks + (p >> 4)];
    if (blk >= 0 && blk < a.num_blocks && blk < kMaxSlotBlocks)
      slot = (int64_t)blk * kPage + (p & (kPage - 1));
  }
  if (threadIdx.x == 0 && a.slots) a.slots[t] = (int32_t)slot;
  // All 16 lanes of a row share j, so the DPP below only reads lanes of the
  // same active row.
  for (int j = threadIdx.x >> 4; j < per_tok; j += blockDim.x / 16) {
    // j in [0, Hq): q head; then the k heads; then the v heads
    if (j >= a.Hq + a.Hkv) {                 // v: a bit copy into the page slot
      const int h = j - a.Hq - a.Hkv;
      if (slot >= 0 && p >= 0 && p < a.max_pos) {
        const int64_t row = slot * a.Hkv + h;   // (page, slot) then KV head
        a.v_cache[row * 16 + sub] = a.v_in[((int64_t)t * a.Hkv + h) * 16 + sub];
      }
      continue;
    }
    const bool is_q = j < a.Hq;
    const int h = is_q ? j : j - a.Hq;
    const u32x4 w = is_q ? a.q_in[((int64_t)t * a.Hq + h) * 16 + sub]
                         : a.k_in[((int64_t)t * a.Hkv + h) * 16 + sub];
    const u32x4 nw = (is_q ? a.q_w : a.k_w)[sub];
    float x[8], wt[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16lo(w[i]); x[2 * i + 1] = bf16hi(w[i]);
      wt[2 * i] = bf16lo(nw[i]); wt[2 * i + 1] = bf16hi(nw[i]);
    }
    // rms_norm: float32 mean of squares and rsqrt, (x * inv) -> bf16, * weight -> bf16.
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(x[i], x[i], ss);
    ss = sum16(ss);
    const float inv = 1.0f / sqrtf(ss / (float)kD + a.eps);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = round_bf16(round_bf16(x[i] * inv) * wt[i]);
    // RoPE: partner dims (+-64) from lane sub ^ 8; rotate_half negates the
    // upper half's values when they move to the lower half.
    const bool low = sub < 8;
    const bool pos_ok = p >= 0 && p < a.max_pos;
    u32x4 cw = {0u, 0u, 0u, 0u}, sw = {0u, 0u, 0u, 0u};
    if (pos_ok) { cw = a.cos_t[(int64_t)p * 16 + sub]; sw = a.sin_t[(int64_t)p * 16 + sub]; }
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float o2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float yi = y[2 * i + e];
        const float partner = dpp_f<kDppRowRor8>(yi);
        const float rot = low ? -partner : partner;
        const float c = e ? bf16hi(cw[i]) : bf16lo(cw[i]);
        const float s = e ? bf16hi(sw[i]) : bf16lo(sw[i]);
        o2[e] = round_bf16(round_bf16(yi * c) + round_bf16(rot * s));
      }
      out[i] = pos_ok ? __builtin_bit_cast(uint32_t, bf16x2{(__bf16)o2[0], (__bf16)o2[1]})
                    : 0x7fc07fc0u;
    }
    const u32x4 ov = {out[0], out[1], out[2], out[3]};
    if (is_q) {
      reinterpret_cast<u32x4*>(a.q_out)[((int64_t)t * a.Hq + h) * 16 + sub] = ov;
    } else if (slot >= 0 && pos_ok) {
      const int64_t row = slot * a.Hkv + h;
      a.k_cache[row * 16 + sub] = ov;
    }
  }
}

}  // namespace

hipError_t launch_qk_norm_rope_append(void* q_out, const void* q_in, const void* k_in,
                                      const void* v_in, const void* q_norm_w,
                                      const void* k_norm_w, const void* cos_table,
                                      const void* sin_table, int max_pos,
                                      const int32_t* block_tables, const int32_t* cu_new,
                                      const int32_t* ctx_lens, int32_t* slots, void* k_cache,
                                      void* v_cache, int B, int max_blocks, int T,
                                      int num_blocks, int Hq, int Hkv, float eps,
                                      hipStream_t stream) {
  if (T == 0) return hipSuccess;
  QkRopeArgs a;
  a.q_out = static_cast<uint16_t*>(q_out);
  a.q_in = static_cast<const u32x4*>(q_in);
  a.k_in = static_cast<const u32x4*>(k_in);
  a.v_in = static_cast<const u32x4*>(v_in);
  a.q_w = static_cast<const u32x4*>(q_norm_w);
  a.k_w = static_cast<const u32x4*>(k_norm_w);
  a.cos_t = static_cast<const u32x4*>(cos_table);
  a.sin_t = static_cast<const u32x4*>(sin_table);
  a.block_tables = block_tables;
  a.cu_new = cu_new;
  a.ctx_lens = ctx_lens;
  a.slots = slots;
  a.k_cache = static_cast<u32x4*>(k_cache);
  a.v_cache = static_cast<u32x4*>(v_cache);
  a.B = B; a.max_blocks = max_blocks; a.T = T; a.num_blocks = num_blocks;
  a.Hq = Hq; a.Hkv = Hkv; a.max_pos = max_pos; a.eps = eps;
  hipLaunchKernelGGL(qk_norm_rope_append_kernel, dim3((unsigned)T), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
