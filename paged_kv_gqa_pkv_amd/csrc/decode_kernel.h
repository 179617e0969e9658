// Decode attention over a paged KV cache, gfx950.
//
// What is computed (Module 04 page, section 1: o_n = softmax(q_n K^T /
// sqrt(d_head)) V over the cached positions; Module 12 page, model.py
// forward with T = 1, query heads grouped as q.view(T, n_kv, group, D)):
// for every sequence b and query head h the softmax-weighted sum of the V
// rows of KV head h / G over positions 0 .. context_lens[b]-1.
//
// Decomposition.  One workgroup owns one (sequence b, context split, group
// of heads_per_wg KV heads) and serves all G = Hq/Hkv query heads of each
// KV head from the same loaded K/V rows, so every K/V byte is read from HBM
// once per step.  Each KV head has `parts` waves, which take disjoint page
// ranges of the split.  Pages are
// stored token-major as in the Module 12 page's paged.py ([page][16 slots][KV
// head][D]), so a 16-token page of one head is 16 rows of 256 B, Hkv*256 B
// apart: lane l holds rows (l>>3) and (l>>3)+8 and the 16-byte chunks (l&7)
// and (l&7)+8 of each, so every load instruction moves eight full 128-byte
// lines.  The K/V rows stay in VGPRs (no LDS staging: the reuse
// across the G heads happens inside each lane).  Scores use v_dot2_f32_bf16
// on the packed bf16 data and an 8-lane DPP butterfly finishes each dot
// product; each lane keeps an online-softmax state (fp32 m, l, acc) over its
// rows, with bf16 probabilities in the PV product.  The lane states, then the
// waves (through LDS), are merged at the end with the usual max/rescale rule.
// Pages are software-pipelined: the next group of pages is in flight while
// the current one is reduced.
//
// Long contexts with few (sequence, head) pairs are cut into splits of
// pages_per_split pages (flash-decoding); each split writes its unnormalised
// (m, l, acc) to the workspace, and the last split of a (sequence, head
// group) to finish merges them all in split order, so results are run-to-run
// bit-identical and the whole call is one kernel.
//
// This header holds the device code (and the host-side argument packing)
// shared by the decode launchers and the mixed-step launch.
#pragma once

#include "pkv.h"
#include "pkv_device.h"
#include "pkv_launch.h"

#include <type_traits>

namespace pkv {
namespace dec {
namespace {


// Tuning constants (measured on MI355X; overridable at build time).
#ifndef PKV_DECODE_NT
#define PKV_DECODE_NT 1            // streaming (non-temporal) K/V loads
#endif
#ifndef PKV_DECODE_WG_PER_CU
#define PKV_DECODE_WG_PER_CU 2     // split planner: waves per SIMD the register budget allows
#endif
#ifndef PKV_DECODE_MIN_PPW
#define PKV_DECODE_MIN_PPW 2       // split planner: minimum pages per wave
#endif
#ifndef PKV_DECODE_WG_COST_PAGES
#define PKV_DECODE_WG_COST_PAGES 3 // split planner: fixed workgroup cost, in page-times
#endif
#ifndef PKV_DECODE_MERGE_COST_PAGES
#define PKV_DECODE_MERGE_COST_PAGES 2  // split planner: fixed cost of the split merge, page-times
#endif
#ifndef PKV_DECODE_SPLIT_COST_EIGHTHS
#define PKV_DECODE_SPLIT_COST_EIGHTHS 8  // split planner: cost per split (its arrival), 1/8 page-time
#endif
#ifndef PKV_DECODE_MAX_HG
#define PKV_DECODE_MAX_HG 1        // most KV heads per workgroup
#endif
#ifndef PKV_DECODE_PARTS
#define PKV_DECODE_PARTS 4         // waves per KV head, splitting its pages
#endif
#ifndef PKV_DECODE_WIDE_PPW
#define PKV_DECODE_WIDE_PPW 16     // pages per wave from which workgroups take two KV heads (0: never)
#endif
#ifndef PKV_DECODE_FORCE_PPW
#define PKV_DECODE_FORCE_PPW 0     // > 0: every plan uses this many pages per wave (tuning)
#endif

constexpr int kMaxPagesPerWave = 64;         // one VGPR of page ids per wave
// Waves a workgroup may hold: eight (two per SIMD, so at most 256 registers
// per lane) for every group size.  At G = 8 that holds because both pages'
// policies there keep O in MFMA tiles (about 190 VGPRs); the v_dot2 bf16
// policy's 16 G accumulators per lane would not fit.
constexpr int max_waves_for(int) { return 8; }
#ifndef PKV_DECODE_MFMA_MIN_G
#define PKV_DECODE_MFMA_MIN_G 8    // bf16 pages: group sizes from which decode runs on the matrix cores
#endif

__device__ __forceinline__ u32x4 load_kv(const u32x4* p) {
#if PKV_DECODE_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}
constexpr float kNegInf = -__builtin_inff();

// Split partials are written and read with agent-coherent accesses (the
// last split to finish, possibly on another XCD, merges them).
__device__ __forceinline__ void ws_store2(float* p, float lo, float hi) {
  const uint64_t bits = (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), bits, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}


struct DecodeArgs {
  uint16_t* out;                 // bf16 [B][Hq][D]
  const u32x4* q;                // bf16 [B][Hq][D] as 16-byte chunks
  const u32x4* k_cache;          // bf16 [num_blocks][16][Hkv][D], or int8 codes (same order)
  const u32x4* v_cache;
  const float* k_scales;         // int8 pages: float32 [num_blocks][Hkv][16]
  const float* v_scales;
  const int32_t* block_tables;   // [B][max_blocks]
  const int32_t* ctx_lens;       // [B]
  // Fused append (no ring): each sequence's newest position, context_lens[b]
  // - 1, takes its K/V rows from k_new/v_new (bf16 [B][Hkv][D]) instead of
  // the pool, and the call writes those rows into that position's slot
  // (k_pool/v_pool are the same pools as k_cache/v_cache; over int8 pages
  // the rows are quantised, and ks_pool/vs_pool are k_scales/v_scales).
  const u32x4* k_new;
  const u32x4* v_new;
  u32x4* k_pool;
  u32x4* v_pool;
  float* ks_pool;
  float* vs_pool;
  float* ws_ml;                  // [B][Hq][S][2] (m, l), log2 domain
  float* ws_acc;                 // [B][Hq][S][D]
  int* counters;                 // [B][Hkv / heads_per_wg] arrivals per (sequence, head group)
  int B, Hq, Hkv, num_blocks, max_blocks, splits, pages_per_split;
  int heads_per_wg;              // KV heads per workgroup
  int parts;                     // waves per KV head, each over 1/parts of the split's pages
  int window;                    // > 0: each sequence's pages form a ring of `window` tokens
  float scale_log2;              // scale * log2(e)
};

// Online softmax per lane.  Each lane keeps its own state (m, l, acc) over
// the rows it holds.  m is a reference point, not the exact running max: it
// moves only when a score exceeds it by more than kRescaleSlack (log2 units),
// so exp2(s - m) stays below 2^kRescaleSlack and the accumulator rescale is
// skipped (wave-uniformly) on almost every page.  The probabilities are
// rounded to bf16 (as the attention of the pages does before its PV product)
// and the PV product runs on v_dot2_f32_bf16, pairing the lane's rows r0 and
// r0+8.
constexpr float kRescaleSlack = 8.f;
constexpr uint32_t kBf16PairOne = 0x3f803f80u;  // bf16 (1, 1)

// Raises the lane's reference max for head j if this page's scores need it
// (rescaling acc and l), then returns the reference to subtract.
template <int U>
__device__ __forceinline__ float softmax_ref(const float (&s)[U][2], float& m, float& l,
                                             float (&acc)[16]) {
  float mc = s[0][0];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) mc = fmaxf(mc, s[u][rr]);
  const bool up = mc > m + kRescaleSlack;   // false while all scores are -inf
  if (__builtin_amdgcn_ballot_w64(up) != 0) {
    const float alpha = up ? fast_exp2(m - mc) : 1.f;   // m = -inf gives 0
    m = up ? mc : m;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[d] *= alpha;
  }
  return (m == kNegInf) ? 0.f : m;
}

// One reduce-scatter step of the lane states: exchange with lane ^ (8 << K)
// (row bit K of the lane), keep the upper half of `in` if that bit is set,
// else the lower half, merged with the partner's copy of the same half.
template <int K>
__device__ __forceinline__ float xchg(float x) {
  if constexpr (K == 0)
    return xor8(x);
  else
    return shfl_xor(x, 8 << K);
}
template <int K, int N>
__device__ __forceinline__ void rs_step(float& m, float& l, const float (&in)[N],
                                        float (&out)[N / 2], int r0) {
  const bool hi = (r0 >> K) & 1;
  float send[N / 2];
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    send[i] = hi ? in[i] : in[N / 2 + i];
    out[i] = hi ? in[N / 2 + i] : in[i];
  }
  const float mo = xchg<K>(m), lo = xchg<K>(l);
  const float M = fmaxf(m, mo);
  const float Mu = (M == kNegInf) ? 0.f : M;
  const float wa = fast_exp2(m - Mu), wb = fast_exp2(mo - Mu);
  l = l * wa + lo * wb;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) out[i] = out[i] * wa + xchg<K>(send[i]) * wb;
  m = M;
}

// bf16 pages.  A 16-token page of one head is 16 rows of 256 B, one per slot
// (Hkv rows apart): lane l holds rows r0 = l>>3 and r0+8, and the 16-byte
// chunks c = l&7 and c+8 of each, i.e. head dims 8c..8c+7 and 64+8c..64+8c+7
// (accumulator d < 8 and d >= 8).
struct Bf16Page {
  struct Regs {
    u32x4 k[2][2];   // [row r0 / r0+8][chunk c / c+8]
    u32x4 v[2][2];
  };
  static __device__ __forceinline__ int dim(int c, int d) {
    return d < 8 ? 8 * c + d : 64 + 8 * c + (d - 8);
  }
  // Fused append: sequence b's new K/V rows of head g as row 0 of a page
  // (lanes 0..7 hold chunks c and c + 8; the other rows stay zero), written
  // into `slot` when it is >= 0.
  static __device__ __forceinline__ void new_row(Regs& r, const DecodeArgs& a, int b, int g,
                                                 int lane, int64_t slot) {
    const int r0 = lane >> 3, c = lane & 7;
    const u32x4* kn = a.k_new + ((int64_t)b * a.Hkv + g) * 16;
    const u32x4* vn = a.v_new + ((int64_t)b * a.Hkv + g) * 16;
    r.k[0][0] = kn[c]; r.k[0][1] = kn[c + 8];
    r.v[0][0] = vn[c]; r.v[0][1] = vn[c + 8];
    if (slot >= 0 && r0 == 0) {
      u32x4* kd = a.k_pool + (slot * a.Hkv + g) * 16;
      u32x4* vd = a.v_pool + (slot * a.Hkv + g) * 16;
      kd[c] = r.k[0][0]; kd[c + 8] = r.k[0][1];
      vd[c] = r.v[0][0]; vd[c + 8] = r.v[0][1];
    }
  }
  // q of the G heads: the lane's two 16-byte chunks of each.
  template <int G>
  struct Q {
    uint32_t w[G][8];
  };
  // Per-lane online-softmax state of each head over the lane's rows.
  template <int G>
  struct State {
    float m[G], l[G], acc[G][16];
  };
  template <int G>
  static __device__ __forceinline__ void init(State<G>& st) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      st.m[j] = kNegInf;
      st.l[j] = 0.f;
#pragma unroll
      for (int d = 0; d < 16; ++d) st.acc[j][d] = 0.f;
    }
  }
  // qp: the group's first head (16 chunks per head).
  template <int G>
  static __device__ __forceinline__ void load_q(Q<G>& q, const u32x4* qp, int lane) {
    const int c = lane & 7;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const u32x4 lo = qp[16 * j + c], hi = qp[16 * j + c + 8];
#pragma unroll
      for (int i = 0; i < 4; ++i) { q.w[j][i] = lo[i]; q.w[j][4 + i] = hi[i]; }
    }
  }
  static __device__ __forceinline__ void load(Regs& r, const DecodeArgs& a, int64_t blk, int g,
                                              int lane) {
    const int r0 = lane >> 3, c = lane & 7;
    const int64_t base = ((blk * kPage + r0) * a.Hkv + g) * 16 + c;   // 16 chunks per row
    const int64_t r8 = (int64_t)8 * a.Hkv * 16;                       // row r0 + 8
    const u32x4* kp = a.k_cache + base;
    const u32x4* vp = a.v_cache + base;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      r.k[0][h] = load_kv(kp + 8 * h);
      r.k[1][h] = load_kv(kp + r8 + 8 * h);
      r.v[0][h] = load_kv(vp + 8 * h);
      r.v[1][h] = load_kv(vp + r8 + 8 * h);
    }
  }
  // kMask: the page is the sequence's last, partially filled one; rows >=
  // valid_rows are excluded (score -inf, V forced to 0 so canary data cannot
  // leak).
  template <int G, int U, bool kMask>
  static __device__ __forceinline__ void process(const Regs (&buf)[U], const Q<G>& q,
                                                 State<G>& st, float scale_log2, int lane,
                                                 int valid_rows) {
    const int r0 = lane >> 3;
    const uint32_t (&qw)[G][8] = q.w;
    float (&m)[G] = st.m;
    float (&l)[G] = st.l;
    float (&acc)[G][16] = st.acc;
    float s[G][U][2];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int j = 0; j < G; ++j) {
          float d = 0.f;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(buf[u].k[rr][h][i]),
                                                  as_bf16x2(qw[j][4 * h + i]), d, false);
          d = sum8(d) * scale_log2;
          if (kMask) d = (r0 + 8 * rr < valid_rows) ? d : kNegInf;
          s[j][u][rr] = d;
        }
    bf16x2 pp[U][G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mu = softmax_ref<U>(s[j], m[j], l[j], acc[j]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        pp[u][j] = bf16x2{(__bf16)fast_exp2(s[j][u][0] - mu), (__bf16)fast_exp2(s[j][u][1] - mu)};
        l[j] = __builtin_amdgcn_fdot2_f32_bf16(pp[u][j], as_bf16x2(kBf16PairOne), l[j], false);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool keep0 = !kMask || (r0 < valid_rows);
      const bool keep1 = !kMask || (r0 + 8 < valid_rows);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w0 = keep0 ? buf[u].v[0][h][i] : 0u;   // row r0, dims 2i, 2i+1
          const uint32_t w1 = keep1 ? buf[u].v[1][h][i] : 0u;   // row r0 + 8
          const bf16x2 lo = as_bf16x2(__builtin_amdgcn_perm(w1, w0, 0x05040100u));
          const bf16x2 hi = as_bf16x2(__builtin_amdgcn_perm(w1, w0, 0x07060302u));
          const int d = 8 * h + 2 * i;
#pragma unroll
          for (int j = 0; j < G; ++j) {
            acc[j][d] = __builtin_amdgcn_fdot2_f32_bf16(lo, pp[u][j], acc[j][d], false);
            acc[j][d + 1] = __builtin_amdgcn_fdot2_f32_bf16(hi, pp[u][j], acc[j][d + 1], false);
          }
        }
    }
  }
  // The wave's merged state of each head, two dims per lane: a
  // reduce-scatter over the 8 row groups (lane bits r0 = 0..2).  At step k
  // each lane merges half of its accumulators with those of lane ^ (8 << k)
  // and keeps that half, so after three steps lane (r0, c) holds head dims
  // d0 and d0 + 1 of its 16 (dim(c, .)), d0 = 8 (r0 & 1) + 4 ((r0 >> 1) & 1)
  // + 2 (r0 >> 2).  Returns the first of the two dims; m and l come out the
  // same in every lane.
  template <int G>
  static __device__ __forceinline__ int finish(State<G>& st, float (&m)[G], float (&l)[G],
                                               float (&v2)[G][2], int lane) {
    const int r0 = lane >> 3, c = lane & 7;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float v8[8], v4[4];
      rs_step<0, 16>(st.m[j], st.l[j], st.acc[j], v8, r0);
      rs_step<1, 8>(st.m[j], st.l[j], v8, v4, r0);
      rs_step<2, 4>(st.m[j], st.l[j], v4, v2[j], r0);
      m[j] = st.m[j];
      l[j] = st.l[j];
    }
    return dim(c, 8 * (r0 & 1) + 4 * ((r0 >> 1) & 1) + 2 * (r0 >> 2));
  }
};

// int8 pages (codes with one float32 scale per (slot, head), read as
// code * scale; Module 04 page, kv_cache.py listing, section 5).  A page of
// one head is 16 rows of 128 codes (Hkv*128 B apart) plus 16 K and 16 V
// scales.  Codes are integers in [-127, 127], exact in bf16.
//
// Both products run on the matrix cores.  The K and V rows arrive as in the
// bf16 policy (lane (r0, c) = (l>>3, l&7): 16-byte chunk c of rows r0 and
// r0 + 8, so every load instruction moves eight whole 128-byte lines) and
// pass, one after the other, through a wave-private 2 KB LDS buffer per page.
//  - Scores: S[key][head] = codes[key] . q[head] for the page's 16 keys is
//    four v_mfma_f32_16x16x32_bf16 (16 keys x 16 head columns, G of them
//    used, 32 dims each).  Lane (g4, t) = (l>>4, l&15) reads key row t, dims
//    32 g4 .. +31, from the buffer and gets back S of keys 4 g4 .. 4 g4 + 3
//    for head t.  (Loading that layout straight from memory splits each row
//    over four lanes: half-used lines per instruction, which the counters
//    showed saturating the L1's tag lookups.)
//  - Softmax: the keys' K scales (DPP row broadcasts) turn S into scores.
//    Each head has one reference, kept alike in the four lanes (g4, t) that
//    hold its scores; lane (g4, t) sums head t's probabilities of keys
//    4 g4 .. +3 of every page.
//  - PV: the probabilities times the keys' V scales, rounded to bf16, are
//    already the A operand of v_mfma_f32_16x16x16_bf16 (lane (g4, t): row
//    head t, k = keys 4 g4 .. +3).  One ds_read_b64_tr_b8 gathers the B
//    operands of two 16-dim blocks: in each group of 16 lanes, lane i
//    receives byte i of eight 16-byte rows, row r being the 8-byte pieces
//    that lanes 2r and 2r + 1 address (checked with probe kernels on the
//    part, as were the MFMA layouts and row_newbcast).  Lane (g4, t)
//    addresses keys 4 g4 .. +3 at dims 32 j .. 32 j + 31 and receives the
//    codes (key 4 g4 + e, dim 32 j + t) and (key 4 g4 + e, dim 32 j + 16 + t),
//    e = 0 .. 3.  Eight MFMAs per page accumulate O[head][dim]: lane (g4, t)
//    holds heads 4 g4 .. 4 g4 + 3, one per accumulator register, at dims
//    16 blk + t (blk = 0 .. 7).
template <int n>
__device__ __forceinline__ float row_bcast(float x) {
  return dpp_f<0x150 + n>(x);     // row_newbcast: lane n of each row of 16
}
// Lane n's value of each row of 16, n = 0 .. G-1, for a compile-time G.
template <int G>
__device__ __forceinline__ void row_bcast_all(float x, float (&out)[G]) {
  if constexpr (G > 0) out[0] = row_bcast<0>(x);
  if constexpr (G > 1) out[1] = row_bcast<1>(x);
  if constexpr (G > 2) { out[2] = row_bcast<2>(x); out[3] = row_bcast<3>(x); }
  if constexpr (G > 4) {
    out[4] = row_bcast<4>(x); out[5] = row_bcast<5>(x);
    out[6] = row_bcast<6>(x); out[7] = row_bcast<7>(x);
  }
}
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
#ifndef PKV_I8_LDS_WAVES
#define PKV_I8_LDS_WAVES 8          // waves of an int8 decode workgroup (at most)
#endif
constexpr int kI8LdsWaves = PKV_I8_LDS_WAVES;
constexpr int kI8LdsPages = 2;    // pages per process call (at most)
// The K/V staging buffers, 2 KB per (wave, page): one array per kernel
// (declared in a function that is not a template, so the instantiations of
// the page loop share it).
__device__ __forceinline__ u32x4 (*i8_lds())[kI8LdsPages][kPage * 8] {
  __shared__ u32x4 s_kv[kI8LdsWaves][kI8LdsPages][kPage * 8];
  return s_kv;
}
// Accumulator register i of row g4 belongs to head 4 g4 + i; its rescale
// factor sits in lane 4 g4 + i of the same row (every row holds every
// head's factor).  Rows past the last head hold nothing of use.
template <int G>
__device__ __forceinline__ void head_factors(float a, float (&ai)[4], int lane) {
  static_assert(G <= 8, "two rows of heads at most");
  if constexpr (G <= 4) {
    ai[0] = row_bcast<0>(a); ai[1] = row_bcast<1>(a);
    ai[2] = row_bcast<2>(a); ai[3] = row_bcast<3>(a);
  } else {
    const bool r1 = (lane & 16) != 0;
    ai[0] = r1 ? row_bcast<4>(a) : row_bcast<0>(a);
    ai[1] = r1 ? row_bcast<5>(a) : row_bcast<1>(a);
    ai[2] = r1 ? row_bcast<6>(a) : row_bcast<2>(a);
    ai[3] = r1 ? row_bcast<7>(a) : row_bcast<3>(a);
  }
}
// Max over the 8 lanes of each aligned group of 8.
__device__ __forceinline__ float max8(float x) {
  x = fmaxf(x, dpp_f<kDppQuadSwap1>(x));
  x = fmaxf(x, dpp_f<kDppQuadSwap2>(x));
  return fmaxf(x, dpp_f<kDppHalfMirror>(x));
}
// Quantise a row of 128 bf16 values held 16 per lane by the 8 lanes of a
// group (lo: values 0..7 of the lane's 16, hi: 8..15): the lane's 16 codes,
// and the row's scale in every lane of the group.
__device__ __forceinline__ u32x4 quantize_row16(const u32x4& lo, const u32x4& hi, float& scale) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16lo(lo[i]); x[2 * i + 1] = bf16hi(lo[i]);
    x[8 + 2 * i] = bf16lo(hi[i]); x[9 + 2 * i] = bf16hi(hi[i]);
  }
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(x[i]));
  mx = max8(mx);
  scale = int8_row_scale(mx);
  const float y = 1.0f / scale;
  u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) out[i >> 2] |= int8_code(x[i], scale, y) << (8 * (i & 3));
  return out;
}
__device__ __forceinline__ s16x4 codes_bf16x4(uint32_t w) {
  const bf16x2 lo = {(__bf16)sbyte0(w), (__bf16)sbyte1(w)};
  const bf16x2 hi = {(__bf16)sbyte2(w), (__bf16)sbyte3(w)};
  const uint32_t u[2] = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  return __builtin_bit_cast(s16x4, u);
}

struct Int8Page {
  struct Regs {
    u32x4 k[2];      // rows r0 and r0 + 8: chunk c
    u32x4 v[2];
    float s;         // t < 4: K scale of key 4 g4 + t; t = 4..7: V scale of key 4 g4 + t - 4
  };
  template <int G>
  struct Q {
    bf16x8 b[4];     // head t's q, dims 32 g4 + 8 kk .. +8, per MFMA kk
  };
  template <int G>
  struct State {
    float m, l;      // lane (g4, t): head t's reference; its sum over keys 4 g4 .. +3 of each page
    f32x4v o[8];     // O[head 4 g4 + i][dim 16 blk + t] in o[blk][i]
  };
  template <int G>
  static __device__ __forceinline__ void init(State<G>& st) {
    st.m = kNegInf;
    st.l = 0.f;
#pragma unroll
    for (int b = 0; b < 8; ++b) st.o[b] = f32x4v{0.f, 0.f, 0.f, 0.f};
  }
  template <int G>
  static __device__ __forceinline__ void load_q(Q<G>& q, const u32x4* qp, int lane) {
    const int t = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (t < G) v = qp[16 * t + 4 * g4 + kk];
      q.b[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // The page's base is uniform; each lane adds a small 32-bit byte offset.
  // A page's scales are head-major ([page][KV head][slot]): head g's 16 K
  // scales are one 64-byte run, as are its 16 V scales.
  static __device__ __forceinline__ void load(Regs& r, const DecodeArgs& a, int64_t blk, int g,
                                              int lane) {
    const int r0 = lane >> 3, c = lane & 7, t = lane & 15, g4 = lane >> 4;
    const int64_t row0 = blk * (int64_t)(kPage * a.Hkv);      // the page's first (slot, head) row
    const char* kp = reinterpret_cast<const char*>(a.k_cache) + row0 * kD;
    const char* vp = reinterpret_cast<const char*>(a.v_cache) + row0 * kD;
    const uint32_t o0 = (uint32_t)((r0 * a.Hkv + g) * kD + 16 * c);
    const uint32_t o8 = o0 + (uint32_t)(8 * a.Hkv * kD);     // row r0 + 8
    const uint32_t os = (uint32_t)(4 * (g * kPage + 4 * g4 + (t & 3)));
    r.k[0] = load_kv(reinterpret_cast<const u32x4*>(kp + o0));
    r.k[1] = load_kv(reinterpret_cast<const u32x4*>(kp + o8));
    r.v[0] = load_kv(reinterpret_cast<const u32x4*>(vp + o0));
    r.v[1] = load_kv(reinterpret_cast<const u32x4*>(vp + o8));
    const char* sp = reinterpret_cast<const char*>((t & 4) ? a.v_scales : a.k_scales) + row0 * 4;
    r.s = *reinterpret_cast<const float*>(sp + os);
  }
  // Fused append: sequence b's new K and V rows of head g, quantised as the
  // append kernel quantises them (the same int8_row_scale / int8_code, so
  // codes and scales agree bit for bit), as row 0 of a page: lane c of row
  // group r0 takes dims 16c .. 16c + 15, lanes 0..7 keep the codes (the
  // other rows stay zero), and lanes t = 0 and t = 4 hold the K and V scale
  // where load() puts key 0's.  Written into `slot` when it is >= 0.
  static __device__ __forceinline__ void new_row(Regs& r, const DecodeArgs& a, int b, int g,
                                                 int lane, int64_t slot) {
    const int r0 = lane >> 3, c = lane & 7, t = lane & 15;
    const u32x4* kn = a.k_new + ((int64_t)b * a.Hkv + g) * 16 + 2 * c;
    const u32x4* vn = a.v_new + ((int64_t)b * a.Hkv + g) * 16 + 2 * c;
    float ks, vs;
    const u32x4 kc = quantize_row16(kn[0], kn[1], ks);
    const u32x4 vc = quantize_row16(vn[0], vn[1], vs);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    r.k[0] = r0 == 0 ? kc : zero;
    r.k[1] = zero;
    r.v[0] = r0 == 0 ? vc : zero;
    r.v[1] = zero;
    r.s = (t & 4) ? vs : ks;
    if (slot >= 0 && r0 == 0) {
      const int64_t row = (slot * a.Hkv + g) * kD;               // bytes
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(a.k_pool) + row + 16 * c) = kc;
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(a.v_pool) + row + 16 * c) = vc;
      if (c == 0) {
        const int64_t si = ((slot / kPage) * a.Hkv + g) * kPage + slot % kPage;
        a.ks_pool[si] = ks;
        a.vs_pool[si] = vs;
      }
    }
  }
  template <int G, int U, bool kMask>
  static __device__ __forceinline__ void process(const Regs (&buf)[U], const Q<G>& q,
                                                 State<G>& st, float scale_log2, int lane,
                                                 int valid_rows) {
    static_assert(U <= kI8LdsPages, "LDS pages per wave");
    u32x4 (*s)[kI8LdsPages][kPage * 8] = i8_lds();
    const int wv = uniform(threadIdx.x >> 6);
    const int r0 = lane >> 3, c = lane & 7, t = lane & 15, g4 = lane >> 4;
    // K rows into the buffer, chunk cc of row r at position cc ^ (r & 7)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      s[wv][u][r0 * 8 + (c ^ r0)] = buf[u].k[0];
      s[wv][u][(r0 + 8) * 8 + (c ^ r0)] = buf[u].k[1];
    }
    // a wave's LDS accesses run in order; keep the compiler from moving
    // the reads above the writes of other lanes (and the V writes above
    // the K reads)
    asm volatile("" ::: "memory");
    u32x4 ka[U], kb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ka[u] = s[wv][u][t * 8 + ((2 * g4) ^ (t & 7))];
      kb[u] = s[wv][u][t * 8 + ((2 * g4 + 1) ^ (t & 7))];
    }
    asm volatile("" ::: "memory");
    // V rows into the same buffer, chunk cc of row r at position
    // cc ^ ((r >> 1) & 7): the transposed reads below (16 rows, 32 B each)
    // then fall on every bank twice
#pragma unroll
    for (int u = 0; u < U; ++u) {
      s[wv][u][r0 * 8 + (c ^ (r0 >> 1))] = buf[u].v[0];
      s[wv][u][(r0 + 8) * 8 + (c ^ (4 + (r0 >> 1)))] = buf[u].v[1];
    }
    asm volatile("" ::: "memory");
    const int vkey = 4 * g4 + ((t >> 1) & 3);     // the row this lane addresses
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4v s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4& kw = (kk < 2) ? ka[u] : kb[u];
        const uint32_t w0 = kw[2 * (kk & 1)], w1 = kw[2 * (kk & 1) + 1];
        const bf16x8 a8 = {(__bf16)sbyte0(w0), (__bf16)sbyte1(w0), (__bf16)sbyte2(w0),
                           (__bf16)sbyte3(w0), (__bf16)sbyte0(w1), (__bf16)sbyte1(w1),
                           (__bf16)sbyte2(w1), (__bf16)sbyte3(w1)};
        s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, q.b[kk], s4, 0, 0, 0);
      }
      const float ks[4] = {row_bcast<0>(buf[u].s), row_bcast<1>(buf[u].s),
                           row_bcast<2>(buf[u].s), row_bcast<3>(buf[u].s)};
      const float vs[4] = {row_bcast<4>(buf[u].s), row_bcast<5>(buf[u].s),
                           row_bcast<6>(buf[u].s), row_bcast<7>(buf[u].s)};
      float sc[4];
      bool keep[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        keep[rr] = !kMask || 4 * g4 + rr < valid_rows;
        sc[rr] = keep[rr] ? s4[rr] * (ks[rr] * scale_log2) : kNegInf;
      }
      // the head's reference, raised (wave-uniformly skipped) only when a
      // score in one of its four lanes exceeds it by more than the slack;
      // the new reference is the largest of the four, so it stays alike
      const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      if (__builtin_amdgcn_ballot_w64(t < G && mx > st.m + kRescaleSlack) != 0) {
        float mh = fmaxf(mx, shfl_xor(mx, 16));
        mh = fmaxf(mh, shfl_xor(mh, 32));
        const bool up = mh > st.m + kRescaleSlack;
        const float alpha = up ? fast_exp2(st.m - mh) : 1.f;   // m = -inf gives 0
        st.m = up ? mh : st.m;
        st.l *= alpha;
        float ai[4];
        head_factors<G>(alpha, ai, lane);
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) st.o[b][i] *= ai[i];
      }
      const float mu = (st.m == kNegInf) ? 0.f : st.m;
      float p[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) p[rr] = fast_exp2(sc[rr] - mu);
      st.l += (p[0] + p[1]) + (p[2] + p[3]);
      // PV weights p * V scale; masked keys weigh exactly 0 (their scale
      // may be a NaN canary)
      float wv4[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) wv4[rr] = keep[rr] ? p[rr] * vs[rr] : 0.f;
      const uint32_t wp[2] = {pack_bf16x2(wv4[0], wv4[1]), pack_bf16x2(wv4[2], wv4[3])};
      const s16x4 wa = __builtin_bit_cast(s16x4, wp);
      const char* vb = reinterpret_cast<const char*>(&s[wv][u][0]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int blk = 2 * j + (t >> 3);
        const int off = vkey * 128 + 16 * (blk ^ ((vkey >> 1) & 7)) + 8 * (t & 1);
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vb + off));
        st.o[2 * j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            wa, codes_bf16x4((uint32_t)x[0]), st.o[2 * j], 0, 0, 0);
        st.o[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            wa, codes_bf16x4((uint32_t)x[1]), st.o[2 * j + 1], 0, 0, 0);
      }
    }
  }
  // Every lane takes head j's reference from lane j of its row and the sum
  // of its four rows' sums; O goes through the wave's buffer (whose last
  // reads have been served) to two dims per lane: dims 2 lane, 2 lane + 1.
  template <int G>
  static __device__ __forceinline__ int finish(State<G>& st, float (&m)[G], float (&l)[G],
                                               float (&v2)[G][2], int lane) {
    static_assert(G * kD * 4 <= kI8LdsPages * kPage * 8 * 16, "O fits the wave's buffer");
    const int t = lane & 15, g4 = lane >> 4;
    float ls = st.l + shfl_xor(st.l, 16);
    ls += shfl_xor(ls, 32);
    row_bcast_all<G>(st.m, m);
    row_bcast_all<G>(ls, l);
    float* so = reinterpret_cast<float*>(&i8_lds()[uniform(threadIdx.x >> 6)][0][0]);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (4 * g4 + i < G) {
#pragma unroll
        for (int b = 0; b < 8; ++b) so[(4 * g4 + i) * kD + 16 * b + t] = st.o[b][i];
      }
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(so + j * kD + 2 * lane);
      v2[j][0] = v[0];
      v2[j][1] = v[1];
    }
    asm volatile("" ::: "memory");
    return 2 * lane;
  }
};

// bf16 pages on the matrix cores, for large groups (the v_dot2 policy keeps
// 16 G accumulators per lane, so at G = 8 its registers leave one wave per
// SIMD).  The products and the softmax bookkeeping are those of Int8Page,
// without codes or scales: per page and wave, four v_mfma_f32_16x16x32_bf16
// give S[key][head] (A = K rows read from a wave-private LDS tile, lane
// (g4, t): row t, dims 32 g4 + 8 kk .. +8 for MFMA kk; B = q of head t, the
// same dims, zero for t >= G), and eight v_mfma_f32_16x16x16_bf16 add the
// rounded probabilities times V into O[head][dim] (B operands from
// ds_read_b64_tr_b16: in each group of 16 lanes, lane j + 4k addresses V[key
// 4 g4 + k][16 blk + 4 j .. +4] and lane i receives V[keys 4 g4 .. +3][16 blk
// + i], the layout the prefill kernel's V^T reads rely on).  The rows arrive
// in the v_dot2 policy's registers (full 128-byte lines per load
// instruction) and go through a 4 KB tile per page whose 16-byte chunks are
// swizzled by row, chunk ^ ((r & 7) << 1 | r >> 3): the 16 rows one K read
// instruction touches, and the 8 rows of each half-wave of a V^T read, fall
// on distinct banks.  Rows of a partial page past its last token are zeroed
// before they reach the tile (an unwritten slot may hold NaN, and a zero
// weight times NaN is NaN).  The row sums add the bf16-rounded
// probabilities, the values the PV product uses.
#ifndef PKV_DECODE_B16M_U
#define PKV_DECODE_B16M_U 1        // pages per pipeline stage of the MFMA bf16 policy
#endif
typedef short i16x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4v lds_i16x4v;
// The tiles of one kernel: kPages pages of kWaves waves, 4 KB each (one
// array per kernel: every process<> instantiation of it uses the same
// template arguments).
template <int kWaves, int kPages>
__device__ __forceinline__ u32x4 (*b16_lds())[kPages][kPage * 16] {
  __shared__ u32x4 s_kv[kWaves][kPages][kPage * 16];
  return s_kv;
}
__device__ __forceinline__ int b16_swz(int r) { return ((r & 7) << 1) | (r >> 3); }

struct Bf16MfmaPage {
  using Regs = Bf16Page::Regs;
  template <int G>
  using Q = Int8Page::Q<G>;
  template <int G>
  using State = Int8Page::State<G>;
  template <int G>
  static __device__ __forceinline__ void init(State<G>& st) { Int8Page::init<G>(st); }
  template <int G>
  static __device__ __forceinline__ void load_q(Q<G>& q, const u32x4* qp, int lane) {
    Int8Page::load_q<G>(q, qp, lane);
  }
  static __device__ __forceinline__ void load(Regs& r, const DecodeArgs& a, int64_t blk, int g,
                                              int lane) {
    Bf16Page::load(r, a, blk, g, lane);
  }
  static __device__ __forceinline__ void new_row(Regs& r, const DecodeArgs& a, int b, int g,
                                                 int lane, int64_t slot) {
    Bf16Page::new_row(r, a, b, g, lane, slot);
  }
  template <int G, int U, bool kMask>
  static __device__ __forceinline__ void process(const Regs (&buf)[U], const Q<G>& q,
                                                 State<G>& st, float scale_log2, int lane,
                                                 int valid_rows) {
    static_assert(U <= PKV_DECODE_B16M_U, "tile pages per wave");
    u32x4 (*s)[PKV_DECODE_B16M_U][kPage * 16] = b16_lds<max_waves_for(G), PKV_DECODE_B16M_U>();
    const int wv = uniform(threadIdx.x >> 6);
    const int r0 = lane >> 3, c = lane & 7, t = lane & 15, g4 = lane >> 4;
    const int sw0 = b16_swz(r0), sw8 = b16_swz(r0 + 8);
    // K rows into the tiles (chunk cc of row r at position cc ^ swz(r))
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        s[wv][u][r0 * 16 + ((c + 8 * h) ^ sw0)] = buf[u].k[0][h];
        s[wv][u][(r0 + 8) * 16 + ((c + 8 * h) ^ sw8)] = buf[u].k[1][h];
      }
    }
    // a wave's LDS accesses run in order; keep the compiler from moving the
    // reads above the writes of other lanes (and the V writes above the K
    // reads)
    asm volatile("" ::: "memory");
    u32x4 kt[U][4];
    const int swt = b16_swz(t);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kt[u][kk] = s[wv][u][t * 16 + ((4 * g4 + kk) ^ swt)];
    asm volatile("" ::: "memory");
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool v0 = !kMask || r0 < valid_rows, v8 = !kMask || r0 + 8 < valid_rows;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        s[wv][u][r0 * 16 + ((c + 8 * h) ^ sw0)] = v0 ? buf[u].v[0][h] : zero;
        s[wv][u][(r0 + 8) * 16 + ((c + 8 * h) ^ sw8)] = v8 ? buf[u].v[1][h] : zero;
      }
    }
    asm volatile("" ::: "memory");
    // the lane's V^T address: key 4 g4 + (t >> 2), dims 16 blk + 4 (t & 3)
    const int vkey = 4 * g4 + (t >> 2);
    const int vsw = b16_swz(vkey);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4v s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kt[u][kk]),
                                                     q.b[kk], s4, 0, 0, 0);
      float sc[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const bool keep = !kMask || 4 * g4 + rr < valid_rows;
        sc[rr] = keep ? s4[rr] * scale_log2 : kNegInf;
      }
      const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      if (__builtin_amdgcn_ballot_w64(t < G && mx > st.m + kRescaleSlack) != 0) {
        float mh = fmaxf(mx, shfl_xor(mx, 16));
        mh = fmaxf(mh, shfl_xor(mh, 32));
        const bool up = mh > st.m + kRescaleSlack;
        const float alpha = up ? fast_exp2(st.m - mh) : 1.f;   // m = -inf gives 0
        st.m = up ? mh : st.m;
        st.l *= alpha;
        float ai[4];
        head_factors<G>(alpha, ai, lane);
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) st.o[b][i] *= ai[i];
      }
      const float mu = (st.m == kNegInf) ? 0.f : st.m;
      float p[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) p[rr] = fast_exp2(sc[rr] - mu);
      const uint32_t wp[2] = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      st.l = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wp[0]), as_bf16x2(kBf16PairOne), st.l,
                                             false);
      st.l = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wp[1]), as_bf16x2(kBf16PairOne), st.l,
                                             false);
      const s16x4 wa = __builtin_bit_cast(s16x4, wp);
      const char* vb = reinterpret_cast<const char*>(&s[wv][u][0]) + vkey * 256 + 8 * (t & 1);
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        const int chunk = 2 * blk + ((t & 3) >> 1);
        const i16x4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4v*)(vb + 16 * (chunk ^ vsw)));
        st.o[blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            wa, __builtin_bit_cast(s16x4, x), st.o[blk], 0, 0, 0);
      }
    }
  }
  // As Int8Page::finish, through this policy's tile.
  template <int G>
  static __device__ __forceinline__ int finish(State<G>& st, float (&m)[G], float (&l)[G],
                                               float (&v2)[G][2], int lane) {
    static_assert(G * kD * 4 <= kPage * 16 * 16, "O fits one tile");
    const int t = lane & 15, g4 = lane >> 4;
    float ls = st.l + shfl_xor(st.l, 16);
    ls += shfl_xor(ls, 32);
    row_bcast_all<G>(st.m, m);
    row_bcast_all<G>(ls, l);
    float* so = reinterpret_cast<float*>(
        &b16_lds<max_waves_for(G), PKV_DECODE_B16M_U>()[uniform(threadIdx.x >> 6)][0][0]);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (4 * g4 + i < G) {
#pragma unroll
        for (int b = 0; b < 8; ++b) so[(4 * g4 + i) * kD + 16 * b + t] = st.o[b][i];
      }
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(so + j * kD + 2 * lane);
      v2[j][0] = v[0];
      v2[j][1] = v[1];
    }
    asm volatile("" ::: "memory");
    return 2 * lane;
  }
};

// Workgroup = one (sequence b, context split, group of heads_per_wg KV
// heads); its heads_per_wg * parts waves are (head hw, page part pw), wave
// w = pw * heads_per_wg + hw.  Wave (hw, pw) serves KV head g = group *
// heads_per_wg + hw and its G query heads over part pw of the split's pages
// (pages_per_split / parts consecutive pages).  The lane states of a wave
// are merged by a reduce-scatter (each lane ends with two head dims), the
// parts of a head through LDS.  With splits, the part-0 wave of each head
// writes its unnormalised (m, l, acc) and the last workgroup of (b, head
// group) to finish merges the splits; the number of splits is kept small,
// since arrivals on one counter are serialised by the memory system.
template <class P, int G, int U, int kMaxWaves, bool kAppend>
__device__ __forceinline__ void decode_body(const DecodeArgs a, const int bid) {
  __shared__ int s_last;
  __shared__ float s_part[kMaxWaves][G][kWave][2];   // parts > 0: two dims per lane and head
  __shared__ float s_ml[kMaxWaves][G][2];
  __shared__ int s_bad[kMaxWaves];

  const int HG = a.heads_per_wg;
  const int PW = a.parts;
  const int n_groups = a.Hkv / HG;
  // bid = ((b * S) + split) * n_groups + group
  const int grp = bid % n_groups;
  const int rest = bid / n_groups;
  const int split = rest % a.splits;
  const int b = rest / a.splits;
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int hw = w % HG, pw = w / HG;
  const int g = grp * HG + hw;
  const int S = a.splits;
  const int pps = a.pages_per_split;
  const int ppw = pps / PW;                   // pages per wave (the plan keeps this exact)

  // Everything up to the page loads is independent of the context length, so
  // the length, the page ids and q are fetched in parallel.  The wave's page
  // range is fixed by the plan; ids past the sequence's last page are
  // fetched (they lie inside the table row) but never used.
  const int p0 = split * pps;
  const int wp0 = p0 + pw * ppw;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;
  const int my_id = (lane < ppw && wp0 + lane < a.max_blocks) ? bt[wp0 + lane] : 0;
  typename P::template Q<G> qv;
  P::template load_q<G>(qv, a.q + ((int64_t)b * a.Hq + g * G) * 16, lane);

  // A length outside [0, planned maximum] poisons the outputs of the sequence
  // (the plan covers splits * pages_per_split pages; no read goes past it).
  // Ring paging (Module 04 page, section 4): a ring of `window` tokens holds
  // the last min(n, window) positions, all at or before the query, in ring
  // slots 0 .. min(n, window) - 1; attention does not depend on their order,
  // so the ring is read like a sequence of that many tokens.
  const int n_ctx = a.ctx_lens[b];
  const int n = (a.window > 0 && n_ctx > a.window) ? a.window : n_ctx;
  const bool bad_len = n < 0 || n > a.max_blocks * kPage ||
                       (n + kPage - 1) / kPage > S * pps;

  // Fused append: position n - 1 comes from k_new / v_new (its slot is not
  // read), and the workgroup whose split holds that position's page (the
  // last split if the length is past the plan) writes the rows into the slot
  // and its part-0 waves add the position's key to their state.  The
  // position's table entry is checked as decode checks every page it reads:
  // an invalid one poisons the output (and, as in slot mapping, no row is
  // written).
  typename P::Regs nrow[1] = {};
  const int n_cache = (kAppend && n >= 1) ? n - 1 : n;
  const int n_pages = bad_len ? 0 : (n_cache + kPage - 1) / kPage;
  const int ns = (n_pages + pps - 1) / pps;     // splits holding cached pages
  // the split owning the new position (-1: none); it is >= ns - 1, since the
  // new position's page is at or after the last cached page
  const int app_split =
      (kAppend && n_ctx >= 1) ? min(((n_ctx - 1) / kPage) / pps, S - 1) : -1;
  const bool owns_new = kAppend && !bad_len && split == app_split;   // uniform
  // splits that contribute: 0 .. nsplit - 1
  const int nsplit = (kAppend && !bad_len && app_split >= 0) ? max(ns, app_split + 1) : ns;
  const bool has_new = owns_new && pw == 0;
  bool new_bad = false;
  if constexpr (kAppend) {
    if (split == app_split && pw == 0) {
      const int tp = (n_ctx - 1) / kPage;
      const int id = tp < a.max_blocks ? bt[tp] : -1;
      new_bad = !(id >= 0 && id < a.num_blocks);
      const int64_t slot =
          (!new_bad && id < kMaxSlotBlocks) ? (int64_t)id * kPage + (n_ctx - 1) % kPage : -1;
      P::new_row(nrow[0], a, b, g, lane, slot);
    }
  }
  const int p1 = min(p0 + pps, n_pages);

  const int64_t orow = ((int64_t)b * a.Hq + g * G) * kD;   // this head's first output row
  if (p0 >= p1 && !owns_new) {
    // Nothing to read.  The first split owns the output of an empty or
    // invalid sequence: zeros for an empty context, NaN for a bad length.
    if (split == 0 && pw == 0) {
      for (int e = lane; e < G * kD; e += kWave) a.out[orow + e] = bad_len ? 0x7fc0u : 0u;
    }
    return;
  }

  // This wave's pages: [w0, w1); full pages first, then the sequence's last
  // page if it is partial and falls in range.
  const int w0 = min(wp0, p1);
  const int w1 = min(wp0 + ppw, p1);
  const int n_full = n_cache / kPage;
  const int nfull = max(0, min(w1, n_full) - w0);
  const bool has_tail = (n_cache % kPage) != 0 && n_full >= w0 && n_full < w1;

  typename P::template State<G> st;
  P::template init<G>(st);

  const int id_base = w0 - wp0;               // lane of my_id holding page w0
  int bad = (bad_len || (has_new && new_bad)) ? 1 : 0;
  auto page_id = [&](int j) -> int64_t {
    const int id = __builtin_amdgcn_readlane(my_id, id_base + j);
    const bool ok = id >= 0 && id < a.num_blocks;
    bad |= ok ? 0 : 1;
    return ok ? id : 0;
  };

  // Full pages, U at a time, two groups in flight.  The steady-state loop
  // covers the pairs of groups whose successor exists, so all its loads are
  // unconditional: the load counter sees one order on every path and the wait
  // before reducing a group leaves the next group in flight.  The last one or
  // two groups are reduced after the loop.
  const int ngroups = nfull / U;
  typename P::Regs bufA[U], bufB[U];
  // q, the length and the page ids have all arrived before the page loads
  // start (the ids are needed for the first address anyway), which keeps
  // them out of the loop's in-flight count.
  __builtin_amdgcn_s_waitcnt(0);
  if (ngroups > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) P::load(bufA[u], a, page_id(u), g, lane);
    const int steady = (ngroups - 1) / 2;
    // The scheduling barriers keep each prefetch between the two reductions:
    // issued before the group it overlaps is reduced, and after the group
    // whose registers it reuses is done (else the two groups' registers
    // overlap and the loop needs copies that wait for the prefetch).
    for (int pi = 0; pi < steady; ++pi) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) P::load(bufB[u], a, page_id((2 * pi + 1) * U + u), g, lane);
      __builtin_amdgcn_sched_barrier(0);
      P::template process<G, U, false>(bufA, qv, st, a.scale_log2, lane, kPage);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) P::load(bufA[u], a, page_id((2 * pi + 2) * U + u), g, lane);
      __builtin_amdgcn_sched_barrier(0);
      P::template process<G, U, false>(bufB, qv, st, a.scale_log2, lane, kPage);
    }
    if (ngroups - 2 * steady == 2) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        P::load(bufB[u], a, page_id((2 * steady + 1) * U + u), g, lane);
      P::template process<G, U, false>(bufA, qv, st, a.scale_log2, lane, kPage);
      P::template process<G, U, false>(bufB, qv, st, a.scale_log2, lane, kPage);
    } else {
      P::template process<G, U, false>(bufA, qv, st, a.scale_log2, lane, kPage);
    }
  }
  // Leftover full pages (fewer than U), one at a time.
  for (int j = ngroups * U; j < nfull; ++j) {
    typename P::Regs one[1];
    P::load(one[0], a, page_id(j), g, lane);
    P::template process<G, 1, false>(one, qv, st, a.scale_log2, lane, kPage);
  }
  if (has_tail) {
    typename P::Regs one[1];
    P::load(one[0], a, page_id(n_full - w0), g, lane);
    P::template process<G, 1, true>(one, qv, st, a.scale_log2, lane, n_cache % kPage);
  }
  if constexpr (kAppend) {
    // the new position as a page whose only valid row is row 0 (lanes 0..7)
    if (has_new) P::template process<G, 1, true>(nrow, qv, st, a.scale_log2, lane, 1);
  }

  // The wave's merged state of each head, two head dims per lane (dd and
  // dd + 1), the same (m, l) in every lane.
  float m[G], l[G], v2[G][2];
  const int dd = P::template finish<G>(st, m, l, v2, lane);

  // Merge the page parts of each head through LDS into its part-0 wave.
  if (PW > 1) {
    if (pw > 0) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        s_part[w][j][lane][0] = v2[j][0];
        s_part[w][j][lane][1] = v2[j][1];
        if (lane == 0) { s_ml[w][j][0] = m[j]; s_ml[w][j][1] = l[j]; }
      }
    }
    if (lane == 0) s_bad[w] = bad;
    __syncthreads();
    if (pw > 0) {
      // other waves only take part in the workgroup's barriers from here
      if (S == 1 || nsplit <= 1) return;
    } else {
      for (int q = 1; q < PW; ++q) {
        const int wq = q * HG + hw;
        bad |= s_bad[wq];
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const float mo = s_ml[wq][j][0], lo = s_ml[wq][j][1];
          const float M = fmaxf(m[j], mo);
          const float Mu = (M == kNegInf) ? 0.f : M;
          const float wa = fast_exp2(m[j] - Mu), wb = fast_exp2(mo - Mu);
          l[j] = l[j] * wa + lo * wb;
          v2[j][0] = v2[j][0] * wa + s_part[wq][j][lane][0] * wb;
          v2[j][1] = v2[j][1] * wa + s_part[wq][j][lane][1] * wb;
          m[j] = M;
        }
      }
    }
  }

  const float nan = __builtin_nanf("");
  if (S == 1 || nsplit <= 1) {
    // a single contributing split (split 0): normalise and write the output
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float inv = 1.f / l[j];
      *reinterpret_cast<uint32_t*>(a.out + orow + j * kD + dd) =
          bad ? 0x7fc07fc0u : pack_bf16x2(v2[j][0] * inv, v2[j][1] * inv);
    }
    return;
  }
  if (pw == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int64_t r = ((int64_t)b * a.Hq + g * G + j) * S + split;
      ws_store2(a.ws_acc + r * kD + dd, bad ? nan : v2[j][0], bad ? nan : v2[j][1]);
      if (lane == 0) ws_store2(a.ws_ml + 2 * r, m[j], bad ? nan : l[j]);
    }
  }

  // Split path: the last of the sequence's contributing splits to finish
  // merges all of them (identical whichever split finishes last).  The
  // partials above were written with agent-coherent stores; waiting for
  // their completion before the arrival is counted, and an acquire fence
  // (cache invalidate) before reading them back, orders them without an L2
  // writeback.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int* counter = a.counters + (int64_t)b * n_groups + grp;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             nsplit - 1;
  __syncthreads();
  if (!s_last || pw > 0) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // Each part-0 wave merges its own head's G query heads, online over
  // batches of kBatch splits.  A batch's loads all go out together: its
  // (m, l) pairs (lane u holds split s0 + u) and every lane's two dims of the
  // partial outputs; then the batch's reference max, the rescale of what the
  // earlier batches summed, and the weighted sum in split order.  Addresses
  // past the last split are clamped and weighted 0, so the loads are
  // unconditional.
  constexpr int kBatch = 64 / G;              // 2 * kBatch * G = 128 VGPRs of partials
  float Mr[G], Lr[G], A[G][2];
#pragma unroll
  for (int j = 0; j < G; ++j) { Mr[j] = kNegInf; Lr[j] = 0.f; A[j][0] = A[j][1] = 0.f; }
  for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
    const int cnt = min(kBatch, nsplit - s0);
    f32x2 mlv[G];
    f32x2 v[G][kBatch];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int64_t rs = ((int64_t)b * a.Hq + g * G + j) * S + s0;   // first split of the batch
      mlv[j] = *reinterpret_cast<const f32x2*>(a.ws_ml + 2 * (rs + min(lane, cnt - 1)));
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        v[j][u] = *reinterpret_cast<const f32x2*>(a.ws_acc + (rs + min(u, cnt - 1)) * kD + dd);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float ms = lane < cnt ? mlv[j][0] : kNegInf;
      const float Mn = fmaxf(Mr[j], wave_max(ms));
      const float Mu = (Mn == kNegInf) ? 0.f : Mn;
      const float resc = fast_exp2(Mr[j] - Mu);
      const float wl = lane < cnt ? fast_exp2(ms - Mu) : 0.f;   // weight of split s0 + lane
      Lr[j] = Lr[j] * resc + wave_sum(lane < cnt ? mlv[j][1] * wl : 0.f);
      A[j][0] *= resc;
      A[j][1] *= resc;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float wgt =
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), u));
        A[j][0] = __builtin_fmaf(v[j][u][0], wgt, A[j][0]);
        A[j][1] = __builtin_fmaf(v[j][u][1], wgt, A[j][1]);
      }
      Mr[j] = Mn;
    }
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float inv = 1.f / Lr[j];
    *reinterpret_cast<uint32_t*>(a.out + orow + j * kD + dd) =
        pack_bf16x2(A[j][0] * inv, A[j][1] * inv);
  }
  // Leave the counter at zero for the next call on this workspace.
  if (hw == 0 && lane == 0)
    __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class P, int G, int U, int kMaxWaves, bool kAppend>
__global__ void __launch_bounds__(kMaxWaves * kWave) decode_kernel(const DecodeArgs a) {
  decode_body<P, G, U, kMaxWaves, kAppend>(a, blockIdx.x);
}

// Pages held per pipeline stage, by group size (register budget: two stages
// of U pages, 32 VGPRs per page, next to 16*G accumulators).
#ifndef PKV_DECODE_U_G1
#define PKV_DECODE_U_G1 2
#endif
#ifndef PKV_DECODE_U_G2
#define PKV_DECODE_U_G2 2
#endif
#ifndef PKV_DECODE_U_G4
#define PKV_DECODE_U_G4 1
#endif
#ifndef PKV_DECODE_U_G8
#define PKV_DECODE_U_G8 1
#endif
// int8 pages hold 20 VGPRs per page (codes and scales), so twice the pages fit.
#ifndef PKV_DECODE_I8_U_G1
#define PKV_DECODE_I8_U_G1 2
#endif
#ifndef PKV_DECODE_I8_U_G2
#define PKV_DECODE_I8_U_G2 2
#endif
#ifndef PKV_DECODE_I8_U_G4
#define PKV_DECODE_I8_U_G4 1
#endif
#ifndef PKV_DECODE_I8_U_G8
#define PKV_DECODE_I8_U_G8 1
#endif


// Where the split path keeps its partials and arrival counters.
struct SplitBuffers {
  float* ml;
  float* acc;
  int* counters;
};

// A caller workspace of plan.ws_bytes: (m, l), then acc, then the counters.
SplitBuffers workspace_buffers(const DecodePlan& plan, void* workspace) {
  char* ws = static_cast<char*>(workspace);
  if (plan.splits <= 1 || !ws) return {nullptr, nullptr, nullptr};
  return {reinterpret_cast<float*>(ws), reinterpret_cast<float*>(ws + plan.ws_ml_bytes),
          reinterpret_cast<int*>(ws + plan.ws_ml_bytes + plan.ws_acc_bytes)};
}

DecodeArgs make_args(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const float* k_scales, const float* v_scales,
                     const int32_t* block_tables, const int32_t* ctx_lens, int B, int Hq,
                     int Hkv, int num_blocks, int max_blocks, float scale,
                     const DecodePlan& plan, const SplitBuffers& wsb, int window) {
  DecodeArgs a;
  a.out = static_cast<uint16_t*>(out);
  a.q = static_cast<const u32x4*>(q);
  a.k_cache = static_cast<const u32x4*>(k_cache);
  a.v_cache = static_cast<const u32x4*>(v_cache);
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.block_tables = block_tables;
  a.ctx_lens = ctx_lens;
  a.k_new = a.v_new = nullptr;
  a.k_pool = a.v_pool = nullptr;
  a.ks_pool = a.vs_pool = nullptr;
  const bool split = plan.splits > 1;
  a.ws_ml = split ? wsb.ml : nullptr;
  a.ws_acc = split ? wsb.acc : nullptr;
  a.counters = split ? wsb.counters : nullptr;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.num_blocks = num_blocks; a.max_blocks = max_blocks;
  a.splits = plan.splits; a.pages_per_split = plan.pages_per_split;
  a.heads_per_wg = plan.heads_per_wg;
  a.parts = plan.parts;
  a.window = window;
  a.scale_log2 = scale * 1.4426950408889634f;
  return a;
}

}  // namespace
}  // namespace dec
}  // namespace pkv
