// Device-side helpers shared by the gfx950 kernels (wave64, CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kPage = 16;     // tokens per page
// Slots are int32 (block id * 16 + offset), so only block ids below 2^27
// have one.
constexpr int kMaxSlotBlocks = 1 << 27;
constexpr int kD = 128;       // head dim
constexpr int kWave = 64;     // CDNA wavefront

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// bf16 pair packed in a u32 -> two floats (a bf16 value is the high half of
// the float with the same value, so these are exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even, NaN kept quiet.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// DPP lane moves inside a row of 16 lanes (bound_ctrl: all lanes valid).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               kCtrl, 0xf, 0xf, true));
}
constexpr int kDppQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]  (lane ^ 1)
constexpr int kDppQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]  (lane ^ 2)
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i <-> 7-i within 8
constexpr int kDppRowRor8 = 0x128;     // row_ror:8 (lane ^ 8 within a row of 16)

// Sum over aligned groups of 8 lanes; every lane of the group gets the sum.
__device__ __forceinline__ float sum8(float x) {
  x += dpp_f<kDppQuadSwap1>(x);
  x += dpp_f<kDppQuadSwap2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  return x;
}

// Cross-lane xor shuffles for the 8-, 16- and 32-lane distances.
__device__ __forceinline__ float xor8(float x) { return dpp_f<kDppRowRor8>(x); }
__device__ __forceinline__ float shfl_xor(float x, int m) {
  int src = (int)(threadIdx.x & 63) ^ m;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

// The values of lanes i % 32 and i % 32 + 32, in every lane i, from one
// v_permlane32_swap (a VALU op, no LDS round trip): swapping two copies of
// x exchanges the upper half of one with the lower half of the other.
// Written as asm: the compiler's builtin returns the first result for both.
// The s_nop gives the two wait states the swap needs after a VALU write of
// its operands.
struct Halves {
  float lo, hi;
};
__device__ __forceinline__ Halves halves32(float x) {
  float lo = x, hi = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
  return {lo, hi};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum and max over the 64 lanes of a wave; every lane gets the result.
__device__ __forceinline__ float wave_sum(float x) {
  x = sum8(x);
  x += xor8(x);
  x += shfl_xor(x, 16);
  return x + shfl_xor(x, 32);
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<kDppQuadSwap1>(x));
  x = fmaxf(x, dpp_f<kDppQuadSwap2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  x = fmaxf(x, xor8(x));
  x = fmaxf(x, shfl_xor(x, 16));
  return fmaxf(x, shfl_xor(x, 32));
}

// Signed byte i of w as a float: one SDWA convert.  Written out because the
// compiler otherwise splits it into a shift and a convert and hoists the
// shifts of the next page's codes into the current iteration (a register
// blow-up that also serialises the page pipeline).
#define PKV_SBYTE(n)                                                               \
  __device__ __forceinline__ float sbyte##n(uint32_t w) {                          \
    float r;                                                                       \
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD "     \
        "src0_sel:BYTE_" #n : "=v"(r) : "v"(w));                                   \
    return r;                                                                      \
  }
PKV_SBYTE(0)
PKV_SBYTE(1)
PKV_SBYTE(2)
PKV_SBYTE(3)
#undef PKV_SBYTE
__device__ __forceinline__ float sbyte(uint32_t w, int i) {
  return i == 0 ? sbyte0(w) : i == 1 ? sbyte1(w) : i == 2 ? sbyte2(w) : sbyte3(w);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Append as a row copy (Module 12 page, paged.py PagedKVCache.write: the
// token's K and V rows into its slot; pages token-major, so one token's rows
// for all KV heads are one contiguous run of Hkv*D*2 bytes).  Work item = one
// 16-byte chunk of one token's K or V row; items first, first + stride, ...
// of the n_items = T * 2 * Hkv * chunks_per_head; consecutive items are
// consecutive chunks of a row, so reads and writes are contiguous runs.
// Tokens whose slot is outside [0, num_slots) are skipped.
__device__ __forceinline__ void append_rows(const u32x4* __restrict__ k_new,
                                            const u32x4* __restrict__ v_new,
                                            const int32_t* __restrict__ slots,
                                            u32x4* __restrict__ k_cache,
                                            u32x4* __restrict__ v_cache, int64_t n_items, int Hkv,
                                            int chunks_per_head, int64_t num_slots,
                                            int64_t first, int64_t stride) {
  const int chunks_per_row = Hkv * chunks_per_head;
  for (int64_t i = first; i < n_items; i += stride) {
    const int64_t t = i / (2 * chunks_per_row);
    const int row_item = (int)(i % (2 * chunks_per_row));
    const int which = row_item / chunks_per_row;
    const int r = row_item % chunks_per_row;     // chunk within the token's [Hkv][D] row
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    const u32x4* src = which ? v_new : k_new;
    u32x4* dst = which ? v_cache : k_cache;
    dst[slot * chunks_per_row + r] = src[t * chunks_per_row + r];
  }
}

// The int8 quantiser of one (token, KV head) row, in float32 as the Module
// 04 page's KV8Cache.write does (kv_cache.py listing, section 5):
//   scale = max_d |x_d| / 127 + 1e-8,   code_d = clip(rint(x_d / scale), -127, 127)
// with round half to even.  The quotients x_d / scale are the correctly
// rounded ones without a full division each: with y = 1 / scale correctly
// rounded (one IEEE division per row) and q = x * y, the residual
// e = x - q * scale is exact in an fma and q + e * y rounds to the correctly
// rounded quotient (Markstein's theorem for round-to-nearest division; it
// needs no underflow in the residual, which holds for every |x| >= scale / 2,
// the only quotients that can round to a nonzero code; smaller ones give code
// 0 either way).  Every kernel that quantises uses these two functions, so
// their codes and scales agree bit for bit.
__device__ __forceinline__ float int8_row_scale(float amax) { return amax / 127.0f + 1e-8f; }
__device__ __forceinline__ uint32_t int8_code(float x, float scale, float y) {
  const float q0 = x * y;
  const float e = __builtin_fmaf(-q0, scale, x);
  const float q = __builtin_fmaf(e, y, q0);
  const float c = fminf(fmaxf(__builtin_rintf(q), -127.f), 127.f);
  return (uint32_t)(int32_t)c & 0xffu;
}

}  // namespace pkv
