// Decode attention over a paged KV cache, gfx950.
//
// What is computed (Module 04 page, section 1: o_n = softmax(q_n K^T /
// sqrt(d_head)) V over the cached positions; Module 12 page, model.py
// forward with T = 1, query heads grouped as q.view(T, n_kv, group, D)):
// for every sequence b and query head h the softmax-weighted sum of the V
// rows of KV head h / G over positions 0 .. context_lens[b]-1.
//
// Decomposition.  One workgroup owns one (sequence b, KV head g, context
// split) and serves all G = Hq/Hkv query heads of the group from the same
// loaded K/V rows, so every K/V byte is read from HBM once per step.  The
// workgroup's 4 waves take disjoint page ranges of the split.  Pages are
// stored head-major, so a 16-token page of one head is 16 contiguous rows of
// 256 B (4 KiB): lane l holds rows (l>>3) and (l>>3)+8 and the 16-byte chunks
// (l&7) and (l&7)+8 of each, so every load instruction moves eight full
// 128-byte lines.  The K/V rows stay in VGPRs (no LDS staging: the reuse
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
// (m, l, acc) to the workspace, and the last split of a (sequence, KV head)
// to finish merges them all in split order, so results are run-to-run
// bit-identical and the whole call is one kernel.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

// Tuning constants (measured on MI355X; overridable at build time).
#ifndef PKV_DECODE_NT
#define PKV_DECODE_NT 1            // streaming (non-temporal) K/V loads
#endif
#ifndef PKV_DECODE_WG_PER_CU
#define PKV_DECODE_WG_PER_CU 2     // split planner: workgroups per compute unit
#endif
#ifndef PKV_DECODE_MIN_PPW
#define PKV_DECODE_MIN_PPW 2       // split planner: minimum pages per wave
#endif
#ifndef PKV_DECODE_WG_COST_PAGES
#define PKV_DECODE_WG_COST_PAGES 3 // split planner: fixed workgroup cost, in page-times
#endif


constexpr int kWaves = 4;                    // waves per workgroup
constexpr int kMaxPagesPerWave = 64;         // one VGPR of page ids per wave

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
__device__ __forceinline__ void ws_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


struct DecodeArgs {
  uint16_t* out;                 // bf16 [B][Hq][D]
  const u32x4* q;                // bf16 [B][Hq][D] as 16-byte chunks
  const u32x4* k_cache;          // bf16 [num_blocks][Hkv][16][D]
  const u32x4* v_cache;
  const int32_t* block_tables;   // [B][max_blocks]
  const int32_t* ctx_lens;       // [B]
  float* ws_ml;                  // [B][Hq][S][2] (m, l), log2 domain
  float* ws_acc;                 // [B][Hq][S][D]
  int* counters;                 // [B][Hkv] arrivals per (sequence, KV head); zero between calls
  int B, Hq, Hkv, num_blocks, max_blocks, splits, pages_per_split;
  float scale_log2;              // scale * log2(e)
};

// K and V of one page for this lane: [row r0 / r0+8][chunk c / c+8].
struct PageRegs {
  u32x4 k[2][2];
  u32x4 v[2][2];
};

__device__ __forceinline__ void load_page(PageRegs& r, const DecodeArgs& a, int64_t blk, int g,
                                          int lane_off) {
  const int64_t row_stride = 16;                              // chunks per row
  const int64_t base = (blk * a.Hkv + g) * kPage * 16;        // chunk 0 of row 0, head g
  const u32x4* kp = a.k_cache + base;
  const u32x4* vp = a.v_cache + base;
  const int o8 = (int)(8 * row_stride);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    r.k[0][h] = load_kv(kp + lane_off + 8 * h);
    r.k[1][h] = load_kv(kp + lane_off + o8 + 8 * h);
    r.v[0][h] = load_kv(vp + lane_off + 8 * h);
    r.v[1][h] = load_kv(vp + lane_off + o8 + 8 * h);
  }
}

// Online-softmax update with U pages held in registers.  kMask: the single
// page is the sequence's last, partially filled one; rows >= valid_rows are
// excluded (score -inf, V forced to 0 so canary data cannot leak).
//
// Each lane keeps its own state (m, l, acc) over the rows it holds.  m is a
// reference point, not the exact running max: it moves only when a score
// exceeds it by more than kRescaleSlack (log2 units), so exp2(s - m) stays
// below 2^kRescaleSlack and the accumulator rescale is skipped (wave-uniformly)
// on almost every page.  The probabilities are rounded to bf16 (as the
// attention of the pages does before its PV product) and the PV product and
// the row sum l run on v_dot2_f32_bf16, pairing the lane's rows r0 and r0+8.
constexpr float kRescaleSlack = 8.f;
constexpr uint32_t kBf16PairOne = 0x3f803f80u;  // bf16 (1, 1)

template <int G, int U, bool kMask>
__device__ __forceinline__ void process(const PageRegs (&buf)[U], const uint32_t (&qw)[G][8],
                                        float (&m)[G], float (&l)[G], float (&acc)[G][16],
                                        float scale_log2, int r0, int valid_rows) {
  float s[U][2][G];
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
        s[u][rr][j] = d;
      }
  bf16x2 pp[U][G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float mc = s[0][0][j];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) mc = fmaxf(mc, s[u][rr][j]);
    const bool up = mc > m[j] + kRescaleSlack;   // false while all scores are -inf
    if (__builtin_amdgcn_ballot_w64(up) != 0) {
      const float alpha = up ? fast_exp2(m[j] - mc) : 1.f;   // m = -inf gives 0
      m[j] = up ? mc : m[j];
      l[j] *= alpha;
#pragma unroll
      for (int d = 0; d < 16; ++d) acc[j][d] *= alpha;
    }
    const float mu = (m[j] == kNegInf) ? 0.f : m[j];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      pp[u][j] = bf16x2{(__bf16)fast_exp2(s[u][0][j] - mu), (__bf16)fast_exp2(s[u][1][j] - mu)};
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

// Merge two online-softmax states (m in the log2 domain).
__device__ __forceinline__ void merge_state(float& m, float& l, float* acc, float m2, float l2,
                                            const float* acc2, int n) {
  const float M = fmaxf(m, m2);
  const float Mu = (M == kNegInf) ? 0.f : M;
  const float a = fast_exp2(m - Mu), b = fast_exp2(m2 - Mu);
  l = l * a + l2 * b;
  for (int d = 0; d < n; ++d) acc[d] = acc[d] * a + acc2[d] * b;
  m = M;
}

template <int G, int U>
__global__ void __launch_bounds__(kWaves * kWave)
decode_kernel(const DecodeArgs a) {
  __shared__ float s_acc[kWaves][G][kD];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ int s_bad[kWaves];
  __shared__ int s_last;

  const int bid = blockIdx.x;                 // ((b * S) + split) * Hkv + g
  const int g = bid % a.Hkv;
  const int rest = bid / a.Hkv;
  const int split = rest % a.splits;
  const int b = rest / a.splits;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int r0 = lane >> 3, c = lane & 7;
  const int S = a.splits;
  const int ppw = a.pages_per_split / kWaves;  // pages per wave (the plan keeps this exact)

  // Everything up to the page loads is independent of the context length, so
  // the length, the page ids and q are fetched in parallel.  The wave's page
  // range is fixed by the plan; ids past the sequence's last page are fetched
  // (they lie inside the table row) but never used.
  const int p0 = split * a.pages_per_split;
  const int wp0 = p0 + w * ppw;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;
  const int my_id = (lane < ppw && wp0 + lane < a.max_blocks) ? bt[wp0 + lane] : 0;
  uint32_t qw[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const u32x4* qp = a.q + ((int64_t)b * a.Hq + g * G + j) * 16;
    const u32x4 lo = qp[c], hi = qp[c + 8];
#pragma unroll
    for (int i = 0; i < 4; ++i) { qw[j][i] = lo[i]; qw[j][4 + i] = hi[i]; }
  }

  // A length outside [0, planned maximum] poisons the outputs of the sequence
  // (the plan covers splits * pages_per_split pages; no read goes past it).
  const int n = a.ctx_lens[b];
  const bool bad_len = n < 0 || n > a.max_blocks * kPage ||
                       (n + kPage - 1) / kPage > S * a.pages_per_split;
  const int n_pages = bad_len ? 0 : (n + kPage - 1) / kPage;
  const int p1 = min(p0 + a.pages_per_split, n_pages);

  if (p0 >= p1) {
    // Nothing to read.  The first split owns the output of an empty or
    // invalid sequence: zeros for an empty context, NaN for a bad length.
    if (split == 0) {
      for (int e = tid; e < G * kD; e += kWaves * kWave) {
        const int j = e / kD, d = e % kD;
        a.out[((int64_t)b * a.Hq + g * G + j) * kD + d] = bad_len ? 0x7fc0u : 0u;
      }
    }
    return;
  }

  // This wave's pages: [w0, w1); full pages first, then the sequence's last
  // page if it is partial and falls in range.
  const int w0 = min(wp0, p1);
  const int w1 = min(wp0 + ppw, p1);
  const int n_full = n / kPage;
  const int nfull = max(0, min(w1, n_full) - w0);
  const bool has_tail = (n % kPage) != 0 && n_full >= w0 && n_full < w1;

  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = kNegInf; l[j] = 0.f;
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[j][d] = 0.f;
  }

  const int lane_off = r0 * 16 + c;
  const int id_base = w0 - wp0;               // lane of my_id holding page w0
  int bad = bad_len ? 1 : 0;
  auto page_id = [&](int j) -> int64_t {
    const int id = __builtin_amdgcn_readlane(my_id, id_base + j);
    const bool ok = id >= 0 && id < a.num_blocks;
    bad |= ok ? 0 : 1;
    return ok ? id : 0;
  };

  // Full pages, U at a time, two groups in flight.
  const int ngroups = nfull / U;
  PageRegs bufA[U], bufB[U];
  if (ngroups > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) load_page(bufA[u], a, page_id(u), g, lane_off);
  }
  for (int gi = 0; gi < ngroups; gi += 2) {
    const bool more1 = gi + 1 < ngroups;
    if (more1) {
#pragma unroll
      for (int u = 0; u < U; ++u) load_page(bufB[u], a, page_id((gi + 1) * U + u), g, lane_off);
    }
    process<G, U, false>(bufA, qw, m, l, acc, a.scale_log2, r0, kPage);
    if (more1) {
      if (gi + 2 < ngroups) {
#pragma unroll
        for (int u = 0; u < U; ++u) load_page(bufA[u], a, page_id((gi + 2) * U + u), g, lane_off);
      }
      process<G, U, false>(bufB, qw, m, l, acc, a.scale_log2, r0, kPage);
    }
  }
  // Leftover full pages (fewer than U), one at a time.
  for (int j = ngroups * U; j < nfull; ++j) {
    PageRegs one[1];
    load_page(one[0], a, page_id(j), g, lane_off);
    process<G, 1, false>(one, qw, m, l, acc, a.scale_log2, r0, kPage);
  }
  if (has_tail) {
    PageRegs one[1];
    load_page(one[0], a, page_id(n_full - w0), g, lane_off);
    process<G, 1, true>(one, qw, m, l, acc, a.scale_log2, r0, n % kPage);
  }

  // Merge the 8 lane groups (rows) of the wave: lanes xor 8, 16, 32.
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float t[16];
    float mo = xor8(m[j]), lo = xor8(l[j]);
#pragma unroll
    for (int d = 0; d < 16; ++d) t[d] = xor8(acc[j][d]);
    merge_state(m[j], l[j], acc[j], mo, lo, t, 16);
#pragma unroll
    for (int sh = 16; sh <= 32; sh <<= 1) {
      mo = shfl_xor(m[j], sh); lo = shfl_xor(l[j], sh);
#pragma unroll
      for (int d = 0; d < 16; ++d) t[d] = shfl_xor(acc[j][d], sh);
      merge_state(m[j], l[j], acc[j], mo, lo, t, 16);
    }
  }

  // Merge the waves through LDS.
  if (lane < 8) {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        s_acc[w][j][c * 8 + d] = acc[j][d];
        s_acc[w][j][64 + c * 8 + d] = acc[j][8 + d];
      }
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) { s_m[w][j] = m[j]; s_l[w][j] = l[j]; }
    s_bad[w] = bad;
  }
  __syncthreads();

  int any_bad = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) any_bad |= s_bad[i];
  const float nan = __builtin_nanf("");
  for (int e = tid; e < G * kD; e += kWaves * kWave) {
    const int j = e / kD, d = e % kD;
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) M = fmaxf(M, s_m[i][j]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const float f = fast_exp2(s_m[i][j] - Mu);
      L = __builtin_fmaf(s_l[i][j], f, L);
      A = __builtin_fmaf(s_acc[i][j][d], f, A);
    }
    const int h = g * G + j;
    if (S == 1) {
      const float o = any_bad ? nan : A / L;
      a.out[((int64_t)b * a.Hq + h) * kD + d] = (uint16_t)f32_to_bf16_bits(o);
    } else {
      const int64_t r = ((int64_t)b * a.Hq + h) * S + split;
      ws_store(a.ws_acc + r * kD + d, any_bad ? nan : A);
      if (d == 0) {
        ws_store(a.ws_ml + 2 * r, M);
        ws_store(a.ws_ml + 2 * r + 1, any_bad ? nan : L);
      }
    }
  }
  if (S == 1) return;

  // Split path: the last of the sequence's non-empty splits to finish merges
  // all of them, in split order (identical whichever split finishes last).
  // The partials above were written with agent-coherent stores; waiting for
  // their completion before the arrival is counted, and an acquire fence
  // (cache invalidate) before reading them back, orders them without an L2
  // writeback.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int ns = (n_pages + a.pages_per_split - 1) / a.pages_per_split;
  int* counter = a.counters + (int64_t)b * a.Hkv + g;
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             ns - 1;
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int e = tid; e < G * kD; e += kWaves * kWave) {
    const int j = e / kD, d = e % kD;
    const int64_t rs = ((int64_t)b * a.Hq + g * G + j) * S;
    const float* ml = a.ws_ml + 2 * rs;
    float M = kNegInf;
    for (int s2 = 0; s2 < ns; ++s2) M = fmaxf(M, ml[2 * s2]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float L = 0.f, A = 0.f;
    for (int s2 = 0; s2 < ns; ++s2) {
      const float f = fast_exp2(ml[2 * s2] - Mu);
      L = __builtin_fmaf(ml[2 * s2 + 1], f, L);
      A = __builtin_fmaf(a.ws_acc[(rs + s2) * kD + d], f, A);
    }
    a.out[((int64_t)b * a.Hq + g * G + j) * kD + d] = (uint16_t)f32_to_bf16_bits(A / L);
  }
  // Leave the counter at zero for the next call on this workspace.
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

template <int G, int U>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)(a.B * a.Hkv * a.splits);
  hipLaunchKernelGGL((decode_kernel<G, U>), dim3(grid), dim3(kWaves * kWave), 0, stream, a);
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// Split planner.  Work units are (sequence, KV head) pairs; a workgroup of 4
// waves streams one split of a unit, and PKV_DECODE_WG_PER_CU workgroups fit
// on a compute unit at once (the kernels' register budget), so the grid runs
// in "rounds" of num_cus * PKV_DECODE_WG_PER_CU workgroups.  For each split
// count the planner estimates the time as rounds * (pages per wave + a fixed
// per-workgroup cost) and keeps the cheapest (fewest splits on ties).
// Splits are 4*PKV_DECODE_MIN_PPW .. 256 pages long (at most 64 pages per
// wave: one VGPR of page ids), in multiples of 4 pages (one share per wave).
// Only host-known sizes enter, so no device->host sync is needed.
DecodePlan plan_decode(int B, int Hq, int Hkv, int max_context_len, int num_cus) {
  DecodePlan p{};
  const int max_pages = max(1, (max_context_len + kPage - 1) / kPage);
  const int units = max(1, B * Hkv);
  const int64_t slots = (int64_t)PKV_DECODE_WG_PER_CU * max(1, num_cus);
  const int min_pps = PKV_DECODE_MIN_PPW * kWaves;
  const int max_pps = kMaxPagesPerWave * kWaves;
  int best_s = 1, best_pps = 0;
  int64_t best_cost = -1;
  int last_pps = -1;
  for (int s_try = 1; s_try <= max_pages; ++s_try) {
    int pps = (max_pages + s_try - 1) / s_try;
    pps = (pps + kWaves - 1) / kWaves * kWaves;
    if (pps > max_pps) continue;
    if (pps < min_pps) pps = min_pps;
    if (pps == last_pps) continue;
    last_pps = pps;
    const int splits = (max_pages + pps - 1) / pps;
    const int64_t rounds = ((int64_t)units * splits + slots - 1) / slots;
    const int64_t cost = rounds * (pps / kWaves + PKV_DECODE_WG_COST_PAGES);
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best_s = splits; best_pps = pps; }
    if (pps == min_pps) break;
  }
  p.splits = best_s;
  p.pages_per_split = best_pps;
  if (best_s > 1) {
    p.ws_ml_bytes = align256((size_t)B * Hq * best_s * 2 * sizeof(float));
    p.ws_acc_bytes = align256((size_t)B * Hq * best_s * kD * sizeof(float));
    p.ws_counter_bytes = align256((size_t)B * Hkv * sizeof(int));
  }
  p.ws_bytes = p.ws_ml_bytes + p.ws_acc_bytes + p.ws_counter_bytes;
  return p;
}

hipError_t launch_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* ctx_lens, int B, int Hq,
                         int Hkv, int num_blocks, int max_blocks, float scale,
                         const DecodePlan& plan, void* workspace, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  DecodeArgs a;
  a.out = static_cast<uint16_t*>(out);
  a.q = static_cast<const u32x4*>(q);
  a.k_cache = static_cast<const u32x4*>(k_cache);
  a.v_cache = static_cast<const u32x4*>(v_cache);
  a.block_tables = block_tables;
  a.ctx_lens = ctx_lens;
  char* ws = static_cast<char*>(workspace);
  const bool split = plan.splits > 1;
  a.ws_ml = split ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_acc = split ? reinterpret_cast<float*>(ws + plan.ws_ml_bytes) : nullptr;
  a.counters = split ? reinterpret_cast<int*>(ws + plan.ws_ml_bytes + plan.ws_acc_bytes)
                     : nullptr;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.num_blocks = num_blocks; a.max_blocks = max_blocks;
  a.splits = plan.splits; a.pages_per_split = plan.pages_per_split;
  a.scale_log2 = scale * 1.4426950408889634f;
  switch (Hq / Hkv) {
    case 1: return launch_g<1, PKV_DECODE_U_G1>(a, stream);
    case 2: return launch_g<2, PKV_DECODE_U_G2>(a, stream);
    case 4: return launch_g<4, PKV_DECODE_U_G4>(a, stream);
    case 8: return launch_g<8, PKV_DECODE_U_G8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
