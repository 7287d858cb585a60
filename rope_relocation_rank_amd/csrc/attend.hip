// Relocate-on-read decode attention on gfx950.
//
// "Kamera: KV Cache Multimodal Unificado e Invariante a Posicao para Reuso sem
// Treinamento" (gist.science/pt/paper/2606.23581), §3, production deployment: the
// rebuild runs as a hook in front of the attention kernel.  Here attention reads the
// cached keys and values and never stores the rebuilt ones:
//     K'_t = R(delta_j) K_t + U_K[t] V_K^T,   V'_t = V_t + U_V[t] V_V^T   (chunk j of t)
//     out  = sum_t softmax_t(scale q . K'_t) V'_t
// for one query per layer and query head (decode), query head h reading KV head
// h / group.
//
// The products are re-associated so that no K' or V' element is ever formed:
//     q . K'_t       = (R(-delta_j) q) . K_t + (V_K^T q) . U_K[t]
//     sum_t p_t V'_t = sum_t p_t V_t + V_V (sum_t p_t U_V[t])
// so per token the kernels read K_t, V_t and the two U rows once, and the rank-m terms
// cost one small product per chunk.  Three kernels:
//   attend_prep   per (layer, chunk, KV head): the rotated query R(-delta_j) q and
//                 V_K^T q of each query head, times scale * log2 e (scores in base 2).
//   attend_tiles  per (layer, KV head, token range): 16-token tiles on MFMA.  Scores
//                 S[t][h] = [K_t | U_K[t]] . [q~_h | w_h] with K rows as the A operand
//                 and the prepared queries, split into bf16 high and low parts (|error|
//                 <= 2^-17 relative), as B: 16x16x32 bf16 MFMA, fp32 accumulation.
//                 Online softmax per query head.  Then O^T += V^T P^T and the U_V sums
//                 on 16x16x16 bf16 MFMA, P split into high and low parts, V^T read
//                 from a per-wave LDS copy of the tile.  Each (range, chunk) segment
//                 writes one partial: max, sum, the 128 value sums and the m U_V sums.
//   attend_merge  per (layer, query head): merges the partials, adding V_V times each
//                 partial's U_V sums with that partial's chunk factor.
#include <hip/hip_runtime.h>

#include "kamera_internal.h"
#include "rope_device.h"

namespace kamera {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;      // prep kernel
constexpr int kTileWaves = 8;              // tile kernel: waves (KV heads) per workgroup
constexpr int kD = kAttendDim;
constexpr int kRowPad = 8;                 // bf16 padding of an LDS tile row
constexpr int kVRow = kD + kRowPad;        // LDS row of a V tile
constexpr int kURow = 128 + kRowPad;       // LDS row of a U_V tile (rank <= 128)

__device__ __forceinline__ float bf16_at(const uint16_t* p) {
  return __uint_as_float((uint32_t)*p << 16);
}

// Last chunk j with offsets[j] <= t: the nonempty chunk holding t when the offsets
// cover t (offsets[0] = 0 <= t).
__device__ __forceinline__ int chunk_at(const int64_t* off, int n, int64_t t) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= t) lo = mid;
    else hi = mid;
  }
  return lo;
}

// 2^(x - m) for a running maximum m that may still be -inf (then nothing counts yet).
__device__ __forceinline__ float weight(float x, float m) {
  return m == -INFINITY ? 0.f : exp2f(x - m);
}

__device__ __forceinline__ float max_xor(float v, int x) {
  return fmaxf(v, __shfl_xor(v, x));
}

// ------------------------------------------------------------------ prepared queries

// One workgroup per (layer, chunk, KV head): V_K rows of the head staged in LDS, then
// each query head's rotated query and V_K^T q.
__global__ __launch_bounds__(kThreads) void attend_prep(AttendArgs a) {
  __shared__ __align__(16) uint16_t svk[kD * 128];  // V_K[g * 128 + d][k], rank <= 128
  __shared__ float sqh[kAttendMaxGroup][kD];
  const int tid = threadIdx.x;
  const int H = a.heads, n = a.num_chunks, m = a.rank, gq = a.group, Hq = a.num_q_heads;
  const uint32_t bid = blockIdx.x;
  const int g = (int)(bid % (uint32_t)H);
  const uint32_t lj = bid / (uint32_t)H;
  const int j = (int)(lj % (uint32_t)n);
  const int l = (int)(lj / (uint32_t)n);
  const int r = a.rope_dim, half = r >> 1;
  const int64_t F = (int64_t)H * kD;
  for (int idx = tid; idx < gq * kD; idx += kThreads) {
    const int h = idx / kD, d = idx - h * kD;
    sqh[h][d] = a.q[((int64_t)l * Hq + g * gq + h) * kD + d];
  }
  if (m > 0) {
    // rows g*128 .. g*128+127 of V_K are one contiguous block of 128 * m elements
    const uint16_t* vk = (const uint16_t*)a.V[0] + (((int64_t)l * n + j) * F + (int64_t)g * kD) * m;
    for (int idx = tid; idx < kD * m / 8; idx += kThreads)
      *(u32x4_t*)(svk + 8 * idx) = *(const u32x4_t*)(vk + 8 * idx);
  }
  __syncthreads();
  const int W = kD + m;
  float* out = a.qw + (((int64_t)l * n + j) * Hq + g * gq) * W;
  for (int idx = tid; idx < gq * kD; idx += kThreads) {
    const int h = idx / kD, d = idx - h * kD;
    float v = sqh[h][d];
    if (d < r) {
      const bool il = a.pairing == 1;
      const int i = il ? d >> 1 : (d < half ? d : d - half);
      const bool first = il ? (d & 1) == 0 : d < half;
      const int dp = il ? (d ^ 1) : (first ? d + half : d - half);
      int sec = 0;
#pragma unroll
      for (int k = 0; k < 3; ++k) sec += (k + 1 < a.num_sections && i >= a.sec_end[k]) ? 1 : 0;
      const int64_t dl = a.delta[(int64_t)j * a.num_sections + sec];
      if (dl != 0) {  // R(-delta): the phase of -delta in the rotation's own form
        const float2 cs = phase_of(a.omega[i], -dl);
        const float b = sqh[h][dp];
        v = first ? fmaf(v, cs.x, -(b * cs.y)) : fmaf(v, cs.x, b * cs.y);
      }
    }
    out[(int64_t)h * W + d] = v * a.scale_log2;
  }
  for (int idx = tid; idx < gq * m; idx += kThreads) {
    const int h = idx / m, k = idx - h * m;
    float w = 0.f;
    for (int d = 0; d < kD; ++d) w = fmaf(sqh[h][d], bf16_at(svk + d * m + k), w);
    out[(int64_t)h * W + kD + k] = w * a.scale_log2;
  }
  // The first chunk's workgroups mark every partial slot of their query heads empty;
  // the tile kernel then fills the slots of the segments that exist.
  if (j == 0) {
    float* ws = a.ws + ((int64_t)l * Hq + g * gq) * a.slots * a.slot_floats;
    for (int i = tid; i < gq * a.slots; i += kThreads) ws[(int64_t)i * a.slot_floats + 1] = 0.f;
  }
}

// ------------------------------------------------------------------ token tiles

// Splits fp32 values into bf16 high and low parts (x - hi - lo <= 2^-17 |x|).
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = (__bf16)x[e];
    lo[e] = (__bf16)(x[e] - (float)hi[e]);
  }
}

// One 16-token tile's A-operand rows as loaded: lane (c16, grp) holds 8 consecutive
// features of token tb + c16 per 32-wide step.
template <int MKX>
struct TileRows {
  u32x4_t k[4], v[4], uk[MKX], uv[MKX];
  bool on;  // the lane's token (tb + c16) has a row in the segment
};

// Two mappings of the work, chosen by what measured faster on each layout:
//  - contiguous caches: one workgroup per (layer, token range), one wave per KV head
//    (heads w, w + 8, ... beyond 8).  The waves read the same tokens' rows side by
//    side, so the workgroup streams whole cache rows and the U rows all heads share are
//    read by one CU.  Each wave walks the range tile by tile and writes its own
//    partials.
//  - paged caches: one 4-wave workgroup per (layer, KV head, token range); the waves
//    take tiles w, w + 4, ... and merge through LDS at the end of each segment.
// A segment is the part of the range inside one chunk; each writes one partial slot per
// query head.  MK: 32-wide rank steps (ceil(m / 32)); PAGED: block-table addressing (and
// the second mapping); PF: the next tile's rows are loaded before the current tile is
// worked (the second register tile lowers occupancy, which pays at one rank step only).
template <int MK, bool PAGED, bool PF>
__global__ __launch_bounds__(PAGED ? kThreads : 64 * kTileWaves)
__attribute__((amdgpu_waves_per_eu(PAGED && MK == 2 ? 3 : 1))) void attend_tiles(AttendArgs a) {
  constexpr int MKX = MK > 0 ? MK : 1;
  constexpr int MU = 2 * MK;               // 16-wide rank blocks of the U_V sums
  constexpr int MUX = MU > 0 ? MU : 1;
  constexpr bool ROWS = !PAGED;
  constexpr int kTileBytes = 16 * (kVRow + kURow) * 2;  // per-wave V and U_V tiles
  // Paged mapping: the tiles' LDS is reused for the merge of the four waves.
  constexpr int kMergeFloats = kWaves * kAttendMaxGroup * (2 + kD + 128);
  constexpr int kLdsTiles = ROWS ? kTileWaves * kTileBytes
                                 : (kWaves * kTileBytes > kMergeFloats * 4 ? kWaves * kTileBytes
                                                                            : kMergeFloats * 4);
  // Paged mapping: the four waves run one KV head, so the query-side B operands (high
  // and low parts of the rotated query and of V_K^T q) are the same for all of them and
  // sit once in LDS after the tiles, read per tile instead of held in 48 registers.
  constexpr int kBOps = 8 + 2 * MKX;  // 16-byte operands per lane
  constexpr int kLds = kLdsTiles + (PAGED ? kBOps * 64 * 16 : 0);
  __shared__ __align__(16) unsigned char lds[kLds];
  u32x4_t* sB = (u32x4_t*)(lds + kLdsTiles);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nw = blockDim.x >> 6;
  const int c16 = lane & 15;
  const int grp = lane >> 4;
  uint16_t* sv = (uint16_t*)(lds + wave * kTileBytes);
  uint16_t* su = sv + 16 * kVRow;
  typedef float MergeRow[kAttendMaxGroup][2 + kD + 128];
  MergeRow* sred = (MergeRow*)lds;

  const uint32_t S = (uint32_t)a.splits;
  const uint32_t bid = blockIdx.x;
  // Workgroup order: split fastest, then (paged) KV head, then layer.
  const uint32_t lg = bid / S;
  const int s = (int)(bid - lg * S);
  const int l = ROWS ? (int)lg : (int)(lg / (uint32_t)a.heads);
  // ROWS: wave w runs heads w, w + nw, ...; otherwise the workgroup runs one head.
  const int g_first = ROWS ? wave : (int)(lg - (uint32_t)l * (uint32_t)a.heads);
  const int g_step = ROWS ? nw : a.heads;
  const int ti_first = ROWS ? 0 : wave;
  const int ti_step = ROWS ? 1 : kWaves;
  const int64_t T = a.total_tokens;
  const int64_t t_lo = (int64_t)s * a.split_tokens;
  const int64_t t_hi = min(T, t_lo + (int64_t)a.split_tokens);
  if (t_lo >= t_hi) return;
  const int m = a.rank, gq = a.group, Hq = a.num_q_heads, n = a.num_chunks;
  const int W = kD + m;
  const bool hv = c16 < gq;                // this lane's MFMA column is a real query head
  const uint16_t* ukb = MK > 0 ? (const uint16_t*)a.U[0] + (int64_t)l * T * m + 8 * grp : nullptr;
  const uint16_t* uvb = MK > 0 ? (const uint16_t*)a.U[1] + (int64_t)l * T * m + 8 * grp : nullptr;
  const uint32_t ss0 = (uint32_t)a.slot_stride[0], ss1 = (uint32_t)a.slot_stride[1];
  const uint32_t ps0 = (uint32_t)a.page_stride[0], ps1 = (uint32_t)a.page_stride[1];
  const uint32_t P = (uint32_t)a.page_size;
  const int psh = (P != 0u && (P & (P - 1u)) == 0u) ? __builtin_ctz(P) : -1;

  // Block-table entry of token t (paged), -1 when t lies at or past `end` or its page
  // id is out of range.  A tile's entries are read one tile ahead, so the row loads of
  // a tile never wait on the table.
  auto page_of = [&](int64_t t, int64_t end) -> int32_t {
    if (!PAGED || t >= end) return -1;
    const uint32_t tt = (uint32_t)t;
    const uint32_t pi = psh >= 0 ? tt >> psh : tt / P;
    const int32_t pg = a.block_table[pi];
    return (pg < 0 || pg >= a.num_pages) ? -1 : pg;
  };
  // Row offsets of token t in the K and V channels inside the layer (32-bit: the host
  // checks the extents), given its block-table entry pg when paged; false when the
  // token has no slot.
  auto slot = [&](int64_t t, int32_t pg, uint32_t& off_k, uint32_t& off_v) -> bool {
    const uint32_t tt = (uint32_t)t;
    if constexpr (PAGED) {
      if (pg < 0) return false;
      const uint32_t pi = psh >= 0 ? tt >> psh : tt / P, si = tt - pi * P;
      off_k = (uint32_t)pg * ps0 + si * ss0;
      off_v = (uint32_t)pg * ps1 + si * ss1;
    } else {
      off_k = tt * ss0;
      off_v = tt * ss1;
    }
    return true;
  };

  // All segments of head g over this workgroup's token range.
  auto run_head = [&](const int g) {
    const uint16_t* kb = (const uint16_t*)a.data[0] + (int64_t)l * a.layer_stride[0] +
                         (int64_t)g * a.head_stride[0] + 8 * grp;
    const uint16_t* vb = (const uint16_t*)a.data[1] + (int64_t)l * a.layer_stride[1] +
                         (int64_t)g * a.head_stride[1] + 8 * grp;
    for (int64_t t0 = t_lo; t0 < t_hi;) {
      const int j = chunk_at(a.offsets, n, t0);
      const int64_t s1 = min(t_hi, a.offsets[j + 1]);
      if (s1 <= t0) break;  // offsets that do not cover the range: nothing more here

      // Loads the rows of tile ti (token tb + c16, 8 consecutive features per step);
      // pg is that token's block-table entry when paged.
      auto load = [&](int ti, int32_t pg, TileRows<MKX>& R) {
        const int64_t tr = t0 + 16 * (int64_t)ti + c16;
        uint32_t off_k = 0, off_v = 0;
        const bool row_on = tr < s1 && slot(tr, pg, off_k, off_v);
        R.on = row_on;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          R.k[ks] = u32x4_t{0u, 0u, 0u, 0u};
          R.v[ks] = u32x4_t{0u, 0u, 0u, 0u};
          if (row_on) {
            R.k[ks] = __builtin_nontemporal_load((const u32x4_t*)(kb + off_k + 32 * ks));
            R.v[ks] = __builtin_nontemporal_load((const u32x4_t*)(vb + off_v + 32 * ks));
          }
        }
#pragma unroll
        for (int ku = 0; ku < MKX; ++ku) {
          R.uk[ku] = u32x4_t{0u, 0u, 0u, 0u};
          R.uv[ku] = u32x4_t{0u, 0u, 0u, 0u};
          if (MK > 0 && tr < s1 && 32 * ku + 8 * grp < m) {
            R.uk[ku] = *(const u32x4_t*)(ukb + tr * m + 32 * ku);
            R.uv[ku] = *(const u32x4_t*)(uvb + tr * m + 32 * ku);
          }
        }
      };
      const int ntiles = (int)((s1 - t0 + 15) >> 4);
      auto tile_page = [&](int ti) -> int32_t {
        return ti < ntiles ? page_of(t0 + 16 * (int64_t)ti + c16, s1) : -1;
      };
      TileRows<MKX> cur;
      int32_t pg_cur = tile_page(ti_first);
      if (PF && ti_first < ntiles) {
        load(ti_first, pg_cur, cur);
        pg_cur = tile_page(ti_first + ti_step);
      }

      // B operands: this lane's query head (column c16), features 32 ks + 8 grp ...
      bf16x8_t qh[4], ql[4], wh[MKX], wl[MKX];
      // Operand o of this lane (paged: from LDS).  Every wave writes the same values
      // for the segment, and reads only after its own writes; the previous segment's
      // readers all passed the barrier that ends it.
      auto bop = [&](int o, const bf16x8_t& r) -> bf16x8_t {
        if constexpr (PAGED) return __builtin_bit_cast(bf16x8_t, sB[o * 64 + lane]);
        return r;
      };
      {
        const float* qp = a.qw + (((int64_t)l * n + j) * Hq + g * gq + (hv ? c16 : 0)) * W;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = hv ? qp[32 * ks + 8 * grp + e] : 0.f;
          split8(x, qh[ks], ql[ks]);
        }
#pragma unroll
        for (int ku = 0; ku < MKX; ++ku) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int k = 32 * ku + 8 * grp + e;
            x[e] = (MK > 0 && hv && k < m) ? qp[kD + k] : 0.f;
          }
          split8(x, wh[ku], wl[ku]);
        }
        if constexpr (PAGED) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            sB[ks * 64 + lane] = __builtin_bit_cast(u32x4_t, qh[ks]);
            sB[(4 + ks) * 64 + lane] = __builtin_bit_cast(u32x4_t, ql[ks]);
          }
#pragma unroll
          for (int ku = 0; ku < MKX; ++ku) {
            sB[(8 + ku) * 64 + lane] = __builtin_bit_cast(u32x4_t, wh[ku]);
            sB[(8 + MKX + ku) * 64 + lane] = __builtin_bit_cast(u32x4_t, wl[ku]);
          }
        }
      }

      float mrun = -INFINITY, lrun = 0.f;
      f32x4_t acc[8], uacc[MUX];
#pragma unroll
      for (int f = 0; f < 8; ++f) acc[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < MUX; ++u) uacc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      for (int ti = ti_first; ti < ntiles; ti += ti_step) {
        const int64_t tb = t0 + 16 * (int64_t)ti;
        TileRows<MKX> nxt;
        int32_t pg_nxt;
        if constexpr (PF) {
          // pg_cur holds the entry of tile ti + ti_step here
          if (ti + ti_step < ntiles) load(ti + ti_step, pg_cur, nxt);
          pg_nxt = tile_page(ti + 2 * ti_step);
        } else {
          load(ti, pg_cur, cur);
          pg_nxt = tile_page(ti + ti_step);
        }
        // Scores of tokens tb + 4 grp + i (i < 4) for query head c16.
        f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8_t A = __builtin_bit_cast(bf16x8_t, cur.k[ks]);
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bop(ks, qh[ks]), sc, 0, 0, 0);
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bop(4 + ks, ql[ks]), sc, 0, 0, 0);
        }
#pragma unroll
        for (int ku = 0; ku < MK; ++ku) {
          const bf16x8_t A = __builtin_bit_cast(bf16x8_t, cur.uk[ku]);
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bop(8 + ku, wh[ku]), sc, 0, 0, 0);
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bop(8 + MKX + ku, wl[ku]), sc, 0, 0, 0);
        }
        // The V and U_V rows go to this wave's LDS tile (row c16) for the transposed
        // reads; the wave's previous reads of the tile come before these writes in
        // program order, and LDS accesses of one wave complete in order.
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          *(u32x4_t*)(sv + c16 * kVRow + 32 * ks + 8 * grp) = cur.v[ks];
#pragma unroll
        for (int ku = 0; ku < MK; ++ku)
          if (32 * ku + 8 * grp < m) *(u32x4_t*)(su + c16 * kURow + 32 * ku + 8 * grp) = cur.uv[ku];
        // Mask tokens past the segment or without a slot.  Paged: bit c16 of the ballot
        // (lanes 0..15) says whether token tb + c16 loaded a row.
        float s4[4];
        if constexpr (PAGED) {
          const uint32_t onm = (uint32_t)__ballot(cur.on) & 0xffffu;
#pragma unroll
          for (int i = 0; i < 4; ++i) s4[i] = (onm >> (4 * grp + i)) & 1u ? sc[i] : -INFINITY;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) s4[i] = tb + 4 * grp + i < s1 ? sc[i] : -INFINITY;
        }
        float mt = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
        mt = max_xor(mt, 16);
        mt = max_xor(mt, 32);
        const float mn = fmaxf(mrun, mt);
        const float corr = weight(mrun, mn);
        if (corr != 1.f) {
          lrun *= corr;
#pragma unroll
          for (int f = 0; f < 8; ++f) acc[f] *= corr;
#pragma unroll
          for (int u = 0; u < MUX; ++u) uacc[u] *= corr;
        }
        mrun = mn;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = weight(s4[i], mn);
          lrun += p[i];
        }
        bf16x4_t ph, pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ph[i] = (__bf16)p[i];
          pl[i] = (__bf16)(p[i] - (float)ph[i]);
        }
        // O^T[f][h] += V^T[f][t] P^T[t][h]: A = V^T rows f = 16 fb + c16, tokens 4 grp + i.
#pragma unroll
        for (int fb = 0; fb < 8; ++fb) {
          bf16x4_t A;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            A[i] = __builtin_bit_cast(__bf16, sv[(4 * grp + i) * kVRow + 16 * fb + c16]);
          acc[fb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, ph, acc[fb], 0, 0, 0);
          acc[fb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, pl, acc[fb], 0, 0, 0);
        }
#pragma unroll
        for (int ub = 0; ub < MU; ++ub) {
          if (16 * ub >= m) break;
          bf16x4_t A;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            A[i] = __builtin_bit_cast(__bf16, su[(4 * grp + i) * kURow + 16 * ub + c16]);
          uacc[ub] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, ph, uacc[ub], 0, 0, 0);
          uacc[ub] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, pl, uacc[ub], 0, 0, 0);
        }
        if constexpr (PF) cur = nxt;
        pg_cur = pg_nxt;
      }
      // The four lane groups of a column hold disjoint tokens' sums.
      lrun += __shfl_xor(lrun, 16);
      lrun += __shfl_xor(lrun, 32);

      // The segment's partial for query head c16: lane (c16, grp) holds features
      // 16 fb + 4 grp + i of the value sums and 16 ub + 4 grp + i of the U_V sums.
      if constexpr (ROWS) {
        if (hv) {
          float* sl = a.ws + (((int64_t)l * Hq + g * gq + c16) * a.slots + (s + j)) * a.slot_floats;
          if (grp == 0) {
            sl[0] = mrun;
            sl[1] = lrun;
            sl[2] = __int_as_float(j);
          }
#pragma unroll
          for (int fb = 0; fb < 8; ++fb)
            *(f32x4_t*)(sl + kAttendSlotHead + 16 * fb + 4 * grp) = acc[fb];
#pragma unroll
          for (int ub = 0; ub < MU; ++ub)
            if (16 * ub + 4 * grp < m)
              *(f32x4_t*)(sl + kAttendSlotHead + kD + 16 * ub + 4 * grp) = uacc[ub];
        }
      } else {
        // Merge the four waves' partials through LDS first.
        __syncthreads();  // the tiles' LDS becomes the merge buffer
        if (hv) {
          if (grp == 0) {
            sred[wave][c16][0] = mrun;
            sred[wave][c16][1] = lrun;
          }
#pragma unroll
          for (int fb = 0; fb < 8; ++fb)
#pragma unroll
            for (int i = 0; i < 4; ++i) sred[wave][c16][2 + 16 * fb + 4 * grp + i] = acc[fb][i];
#pragma unroll
          for (int ub = 0; ub < MU; ++ub)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int k = 16 * ub + 4 * grp + i;
              if (k < m) sred[wave][c16][2 + kD + k] = uacc[ub][i];
            }
        }
        __syncthreads();
        for (int idx = tid; idx < gq * W; idx += kThreads) {
          const int h = idx / W, e = idx - h * W;
          float M = -INFINITY;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sred[w][h][0]);
          float L = 0.f, A = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) {
            const float f = weight(sred[w][h][0], M);
            L = fmaf(f, sred[w][h][1], L);
            A = fmaf(f, sred[w][h][2 + e], A);
          }
          float* sl = a.ws + (((int64_t)l * Hq + g * gq + h) * a.slots + (s + j)) * a.slot_floats;
          if (e == 0) {
            sl[0] = M;
            sl[1] = L;
            sl[2] = __int_as_float(j);
          }
          sl[kAttendSlotHead + e] = A;
        }
        __syncthreads();  // the next segment reuses the LDS for tiles
      }
      t0 = s1;
    }
  };
  if constexpr (ROWS) {
    for (int g = g_first; g < a.heads; g += g_step) run_head(g);
  } else {
    run_head(g_first);
  }
}

// ------------------------------------------------------------------ merge

// One workgroup per (layer, query head), thread d.  Slots with a positive sum are the
// segments' partials, in token order, so their chunks come in nondecreasing order:
// the value sums are merged per thread, the U_V sums are merged per chunk and V_V of
// that chunk is applied once when the chunk changes.  Slots are read 8 at a time so
// their loads overlap.
__global__ __launch_bounds__(kD) void attend_merge(AttendArgs a) {
  __shared__ float smax[kD / 64];
  __shared__ float su[128];
  const int Hq = a.num_q_heads;
  const int hq = (int)(blockIdx.x % (uint32_t)Hq);
  const int l = (int)(blockIdx.x / (uint32_t)Hq);
  const int g = hq / a.group;
  const int d = threadIdx.x;
  const int m = a.rank, n = a.num_chunks, ns = a.slots, SF = a.slot_floats;
  const int64_t F = (int64_t)a.heads * kD;
  const float* base = a.ws + ((int64_t)l * Hq + hq) * ns * SF;
  float M = -INFINITY;
  for (int i = d; i < ns; i += kD) {
    const float* sl = base + (int64_t)i * SF;
    if (sl[1] > 0.f) M = fmaxf(M, sl[0]);
  }
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
  if ((d & 63) == 0) smax[d >> 6] = M;
  __syncthreads();
  M = smax[0];
#pragma unroll
  for (int w = 1; w < kD / 64; ++w) M = fmaxf(M, smax[w]);

  float num = 0.f, den = 0.f, uk = 0.f;
  int jcur = -1;
  // Adds V_V[chunk jcur] times the chunk's merged U_V sums to this thread's value.
  auto flush = [&]() {
    __syncthreads();
    if (d < m) su[d] = uk;
    __syncthreads();
    const u32x4_t* vv = (const u32x4_t*)((const uint16_t*)a.V[1] +
                                         (((int64_t)l * n + jcur) * F + (int64_t)g * kD + d) * m);
#pragma unroll 4
    for (int k8 = 0; k8 < m / 8; ++k8) {
      const u32x4_t w = vv[k8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        num = fmaf(__uint_as_float(w[e] << 16), su[8 * k8 + 2 * e], num);
        num = fmaf(__uint_as_float(w[e] & 0xffff0000u), su[8 * k8 + 2 * e + 1], num);
      }
    }
    uk = 0.f;
  };
  constexpr int kB = 8;
  for (int i0 = 0; i0 < ns; i0 += kB) {
    float ls[kB], ms[kB], av[kB], uv[kB];
    int js[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      ls[u] = 0.f;
      ms[u] = 0.f;
      av[u] = 0.f;
      uv[u] = 0.f;
      js[u] = 0;
      if (i0 + u < ns) {
        const float* sl = base + (int64_t)(i0 + u) * SF;
        ls[u] = sl[1];
        ms[u] = sl[0];
        js[u] = __float_as_int(sl[2]);
        av[u] = sl[kAttendSlotHead + d];
        if (d < m) uv[u] = sl[kAttendSlotHead + kD + d];
      }
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      if (!(ls[u] > 0.f)) continue;  // the same for every thread
      if (m > 0 && js[u] != jcur) {
        if (jcur >= 0) flush();
        jcur = js[u];
      }
      const float f = exp2f(ms[u] - M);
      den = fmaf(f, ls[u], den);
      num = fmaf(f, av[u], num);
      uk = fmaf(f, uv[u], uk);
    }
  }
  if (m > 0 && jcur >= 0) flush();
  const int64_t o = (int64_t)l * Hq + hq;
  a.out[o * kD + d] = den > 0.f ? num / den : 0.f;
  if (a.lse != nullptr && d == 0)
    a.lse[o] = den > 0.f ? (M + log2f(den)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.splits > 0) {  // no tokens: only the merge runs, writing 0 and -inf
    const dim3 grid0((unsigned)((int64_t)a.num_layers * a.num_chunks * a.heads));
    hipLaunchKernelGGL(attend_prep, grid0, dim3(kThreads), 0, s, a);
    // Contiguous: a workgroup per (layer, split), a wave per KV head; paged: a 4-wave
    // workgroup per (layer, split, KV head).
    const bool rows = a.page_size == 0;
    const dim3 grid1((unsigned)((int64_t)a.num_layers * a.splits * (rows ? 1 : a.heads)));
    const dim3 block1((unsigned)(rows ? 64 * (a.heads < kTileWaves ? a.heads : kTileWaves) : kThreads));
    const int mk = (a.rank + 31) / 32;
#define KAMERA_ATT(MK)                                                                   \
  do {                                                                                   \
    if (a.page_size > 0)                                                                 \
      hipLaunchKernelGGL((attend_tiles<MK, true, MK == 1>), grid1, block1, 0, s, a);   \
    else                                                                                 \
      hipLaunchKernelGGL((attend_tiles<MK, false, MK == 1>), grid1, block1, 0, s, a);  \
  } while (0)
    if (mk == 0) KAMERA_ATT(0);
    else if (mk == 1) KAMERA_ATT(1);
    else if (mk == 2) KAMERA_ATT(2);
    else KAMERA_ATT(4);
#undef KAMERA_ATT
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid2((unsigned)((int64_t)a.num_layers * a.num_q_heads));
  hipLaunchKernelGGL(attend_merge, grid2, dim3(kD), 0, s, a);
  return hipGetLastError();
}

}  // namespace kamera
