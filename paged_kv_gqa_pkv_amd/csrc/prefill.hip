// Causal chunked-prefill attention over a paged KV cache on bf16 MFMA, gfx950.
//
// What is computed (Module 12 page, model.py forward with T > 1: scores
// q K^T / sqrt(D) over the cached prefix plus the chunk, mask kpos <= qpos on
// absolute positions, softmax in fp32, probabilities times V; the chunk's
// K/V are appended before the call): for every query row of the chunk, the
// softmax-weighted sum of the V rows of its KV head over keys 0 .. its
// position.
//
// Decomposition.  The G = Hq/Hkv query heads of one KV head are stacked as
// extra rows (row R <-> token R / G, head R % G), so each K/V tile is used by
// all of them.  A workgroup of 4 waves owns 128 such rows of one (sequence,
// KV head); each wave owns 32 rows.  Keys are walked in tiles of 64 (four
// pages, gathered through the block table) that all 4 waves share through
// LDS, double-buffered so the next tile's global loads overlap the current
// tile's MFMA work.
//
// Per tile and wave, on v_mfma_f32_32x32x16_bf16:
//   S^T[keys x rows] = K[keys x D] . Q^T[D x rows]   (2 key blocks x 8 k-steps)
//   O^T[D x rows]   += V^T[D x keys] . P^T[keys x rows] (4 dim blocks x 4 k-steps)
// Computing the transposed products puts one query row in each lane column,
// so the row max is a lane-local max plus one exchange with lane ^ 32, and
// the S^T accumulator registers are already the B operand of the PV product
// (the k index order inside an MFMA is free as long as both operands agree).
// Softmax statistics stay in fp32; P is rounded to bf16 only as an MFMA
// operand, and the row sums use the same rounded values.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerWG = kWaves * kRowsPerWave;   // 128
constexpr int kTileKeys = 64;                       // 4 pages
constexpr int kKStride = kD * 2 + 16;               // bytes per LDS key row (padded)
constexpr int kTileBytes = kTileKeys * kKStride;    // one K or V tile in LDS
constexpr float kNegInf = -__builtin_inff();

struct PrefillArgs {
  uint16_t* out;                 // bf16 [total_q][Hq][D]
  const u32x4* q;                // bf16 [total_q][Hq][D] as 16-byte chunks
  const int32_t* cu_q;           // [B+1]
  const u32x4* k_cache;          // bf16 [num_blocks][16][Hkv][D]
  const u32x4* v_cache;
  const int32_t* block_tables;   // [B][max_blocks]
  const int32_t* ctx_lens;       // [B]
  int B, total_q, max_q_len, Hq, Hkv, G, num_blocks, max_blocks, qtiles;
  float scale_log2;
};

// One thread's share of a tile: 4 chunks of K and 4 of V (16 B each).
struct TileRegs {
  u32x4 k[4];
  u32x4 v[4];
};

// Thread t loads chunk (t & 15) of key rows (t >> 4) + 16*i, i = 0..3, so 16
// consecutive threads read one 256-byte row.  Keys at or past `n` (the
// context length) or past the table are zero-filled: they are always masked,
// and zeros keep canary NaNs out of the products.
__device__ __forceinline__ void load_tile(TileRegs& r, const PrefillArgs& a, const int32_t* bt,
                                          int key0, int n, int g, int tid, int& bad) {
  const int chunk = tid & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = key0 + (tid >> 4) + 16 * i;
    u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (key < n) {
      int blk = bt[key >> 4];
      if (blk < 0 || blk >= a.num_blocks) { bad = 1; blk = 0; }
      const int64_t idx = (((int64_t)blk * kPage + (key & 15)) * a.Hkv + g) * 16 + chunk;
      kv = __builtin_nontemporal_load(a.k_cache + idx);
      vv = __builtin_nontemporal_load(a.v_cache + idx);
    }
    r.k[i] = kv;
    r.v[i] = vv;
  }
}

__device__ __forceinline__ void store_tile(const TileRegs& r, char* ks, char* vs, int tid) {
  const int chunk = tid & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = (tid >> 4) + 16 * i;
    *reinterpret_cast<u32x4*>(ks + key * kKStride + chunk * 16) = r.k[i];
    *reinterpret_cast<u32x4*>(vs + key * kKStride + chunk * 16) = r.v[i];
  }
}

__global__ void __launch_bounds__(kWaves * kWave)
prefill_kernel(const PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char s_k[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) char s_v[2][kTileBytes];
  __shared__ int s_bad;

  const int bid = blockIdx.x;                 // ((b * qtiles) + x) * Hkv + g
  const int g = bid % a.Hkv;
  const int rest = bid / a.Hkv;
  const int x = a.qtiles - 1 - (rest % a.qtiles);   // heaviest (latest) row tiles first
  const int b = rest / a.qtiles;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int G = a.G;

  const int q_lo_raw = a.cu_q[b];
  const int T_raw = a.cu_q[b + 1] - q_lo_raw;
  const int n = a.ctx_lens[b];
  // Rows outside [0, total_q) or more than max_q_len of them: nothing is read
  // or written for this sequence (its rows, if any exist, are not ours).
  if (q_lo_raw < 0 || T_raw < 0 || q_lo_raw + T_raw > a.total_q || T_raw > a.max_q_len) return;
  const int q_lo = q_lo_raw, T = T_raw;
  const int R0 = x * kRowsPerWG;
  if (R0 >= T * G) return;                    // uniform over the workgroup
  const bool bad_len = T > n || n > a.max_blocks * kPage;

  // This lane's query row (lane column of the MFMA tiles).
  const int row = R0 + w * kRowsPerWave + (lane & 31);
  const int t_row = row / G, j_row = row % G;
  const bool row_ok = t_row < T;
  const int qpos = row_ok ? n - T + t_row : -1;
  const int half = lane >> 5;                 // which 8 of 16 k values the lane holds

  // Q^T as the B operand: lane holds Q[row][16ks + 8*half .. +8], ks = 0..7.
  bf16x8 qb[8];
  {
    const u32x4* qp = a.q + ((int64_t)(q_lo + t_row) * a.Hq + g * G + j_row) * 16;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok && !bad_len) v = qp[2 * ks + half];
      qb[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Keys this workgroup needs: 0 .. the last position of its rows.
  const int t_last = min(T - 1, (R0 + kRowsPerWG - 1) / G);
  const int key_end = bad_len ? 0 : n - T + t_last + 1;
  const int n_tiles = (key_end + kTileKeys - 1) / kTileKeys;
  const int t_first = R0 / G;
  const int qpos_min = n - T + t_first;       // smallest position in the workgroup
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m = kNegInf, l = 0.f;
  int bad = 0;

  TileRegs tr;
  if (n_tiles > 0) {
    load_tile(tr, a, bt, 0, key_end, g, tid, bad);
    store_tile(tr, s_k[0], s_v[0], tid);
  }
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int cur = it & 1;
    const int key0 = it * kTileKeys;
    const bool more = it + 1 < n_tiles;
    if (more) load_tile(tr, a, bt, key0 + kTileKeys, key_end, g, tid, bad);

    const char* ks = s_k[cur];
    const char* vs = s_v[cur];

    // S^T = K . Q^T for the two 32-key blocks of the tile.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
      const char* krow = ks + (kb * 32 + (lane & 31)) * kKStride + half * 16;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + kk * 32);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[kk], s[kb], 0, 0, 0);
      }
    }

    // Scale, causal mask, running max.  Accumulator i of block kb holds key
    // key0 + 32*kb + 8*(i/4) + 4*half + i%4.
    const bool need_mask = key0 + kTileKeys - 1 > qpos_min;
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = s[kb][i] * a.scale_log2;
        if (need_mask) {
          const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
          v = key <= qpos ? v : kNegInf;
        }
        s[kb][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float mu = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m - mu);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;

    // P^T in bf16: B operand of the PV product, k-step (kb, hh) = registers
    // 8*hh .. 8*hh+7 of block kb.
    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const __bf16 p = (__bf16)fast_exp2(s[kb][i] - mu);
        pb[kb][i >> 3][i & 7] = p;
        l += (float)p;
      }

    // O^T += V^T . P^T.  The A operand for dim block db, k-step (kb, hh):
    // lane holds V[key][32*db + lane%32] for the 8 keys
    // key0 + 32*kb + 16*hh + 8*(e/4) + 4*half + e%4, e = 0..7.
    const uint16_t* vcol = reinterpret_cast<const uint16_t*>(vs) + (lane & 31);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int kbase = 32 * kb + 16 * hh + 4 * half;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          bf16x8 va;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = kbase + 8 * (e >> 2) + (e & 3);
            va[e] = __builtin_bit_cast(__bf16, vcol[key * (kKStride / 2) + 32 * db]);
          }
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb][hh], o[db], 0, 0, 0);
        }
      }

    if (more) store_tile(tr, s_k[cur ^ 1], s_v[cur ^ 1], tid);
    __syncthreads();
  }

  // Row sums: each half of the lanes summed its own keys.
  l += shfl_xor(l, 32);
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (bad) s_bad = 1;
  __syncthreads();
  if (!row_ok) return;
  const bool poisoned = bad_len || s_bad;
  const float inv = 1.f / l;
  uint32_t* orow = reinterpret_cast<uint32_t*>(
      a.out + ((int64_t)(q_lo + t_row) * a.Hq + g * G + j_row) * kD);
  // O^T accumulator i of dim block db holds dim 32*db + 8*(i/4) + 4*half + i%4.
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = 32 * db + 8 * i4 + 4 * half;
      float v0 = o[db][4 * i4 + 0] * inv, v1 = o[db][4 * i4 + 1] * inv;
      float v2 = o[db][4 * i4 + 2] * inv, v3 = o[db][4 * i4 + 3] * inv;
      uint32_t w0 = pack_bf16x2(v0, v1), w1 = pack_bf16x2(v2, v3);
      if (poisoned) { w0 = 0x7fc07fc0u; w1 = 0x7fc07fc0u; }
      orow[d0 / 2] = w0;
      orow[d0 / 2 + 1] = w1;
    }
}

}  // namespace

hipError_t launch_prefill(void* out, const void* q, const int32_t* cu_q, const void* k_cache,
                          const void* v_cache, const int32_t* block_tables,
                          const int32_t* ctx_lens, int B, int total_q, int max_q_len, int Hq,
                          int Hkv, int num_blocks, int max_blocks, float scale,
                          hipStream_t stream) {
  if (B == 0 || total_q == 0 || max_q_len == 0) return hipSuccess;
  PrefillArgs a;
  a.out = static_cast<uint16_t*>(out);
  a.q = static_cast<const u32x4*>(q);
  a.cu_q = cu_q;
  a.k_cache = static_cast<const u32x4*>(k_cache);
  a.v_cache = static_cast<const u32x4*>(v_cache);
  a.block_tables = block_tables;
  a.ctx_lens = ctx_lens;
  a.B = B; a.total_q = total_q; a.max_q_len = max_q_len;
  a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.num_blocks = num_blocks; a.max_blocks = max_blocks;
  a.qtiles = (max_q_len * a.G + kRowsPerWG - 1) / kRowsPerWG;
  a.scale_log2 = scale * 1.4426950408889634f;
  const unsigned grid = (unsigned)((int64_t)B * a.qtiles * Hkv);
  hipLaunchKernelGGL(prefill_kernel, dim3(grid), dim3(kWaves * kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
