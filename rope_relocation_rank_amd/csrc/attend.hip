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
//     q . K'_t   = (R(-delta_j) q) . K_t + (V_K^T q) . U_K[t]
//     sum_t p_t V'_t = sum_t p_t V_t + V_V (sum_t p_t U_V[t])
// The rotated query and V_K^T q are built once per (split, chunk) segment; per token the
// kernel reads K_t, V_t and the two U rows once (the bytes an attention kernel reads
// anyway plus 4m bytes), and the rank-m tail of the output is one V_V product per
// segment.  The relocate + patch pass that would otherwise write K' and V' back to HBM
// and the re-read of them disappear.  All arithmetic is fp32 on exactly converted bf16
// inputs; scores are kept in base 2 (scale * log2 e folded into the query).
//
// Work split (flash-decoding): tokens are cut into `splits` ranges per (layer, KV head);
// a workgroup (4 waves, 8 row groups of 32 lanes, lane c holding features 4c..4c+3)
// streams its range, cut again at chunk boundaries, with an online softmax per row
// group; the row groups are merged at the end of each segment, which writes one partial
// (max, sum, 128 partial sums) per query head.  A second kernel merges the partials of
// each (layer, query head).
#include <hip/hip_runtime.h>

#include "kamera_internal.h"
#include "rope_device.h"

namespace kamera {
namespace {

typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowGroups = 2 * kWaves;  // 32 lanes per token row
constexpr int kD = kAttendDim;

__device__ __forceinline__ float bf16_at(const uint16_t* p) {
  return __uint_as_float((uint32_t)*p << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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

// Sum over the 32 lanes of each half-wave; every lane of the wavefront calls it.
__device__ __forceinline__ float sum32(float v) {
  v += __uint_as_float(lane_xor<1>(__float_as_uint(v)));
  v += __uint_as_float(lane_xor<2>(__float_as_uint(v)));
  v += __uint_as_float(lane_xor<4>(__float_as_uint(v)));
  v += __uint_as_float(lane_xor<8>(__float_as_uint(v)));
  v += __uint_as_float(lane_xor<16>(__float_as_uint(v)));
  return v;
}

// 2^(x - m) for a running maximum m that may still be -inf (then nothing counts yet).
__device__ __forceinline__ float weight(float x, float m) {
  return m == -INFINITY ? 0.f : exp2f(x - m);
}

// G: query heads per KV head the kernel is built for (the group may be smaller);
// MU: U entries per lane (rank <= 32 MU); NB: token rows per row group per step;
// PAGED: block-table addressing.
template <int G, int MU, int NB, bool PAGED>
__global__ __launch_bounds__(kThreads) void attend_split(AttendArgs a) {
  constexpr int MUX = MU > 0 ? MU : 1;
  __shared__ float sq[G][kD];               // rotated query * scale * log2 e
  __shared__ float sw[G][kD];               // V_K^T q * scale * log2 e (rank <= 128)
  __shared__ float sred[kWaves][G][2 + 2 * kD];  // per wave: max, sum, 128 sums, U_V sums
  __shared__ float sub[G][kD];              // merged U_V sums
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane & 31;
  const int rg = wave * 2 + (lane >> 5);
  const uint32_t S = (uint32_t)a.splits;
  const uint32_t bid = blockIdx.x;
  const int s = (int)(bid % S);
  const uint32_t rest = bid / S;
  const int g = (int)(rest % (uint32_t)a.heads);
  const int l = (int)(rest / (uint32_t)a.heads);
  const int64_t T = a.total_tokens;
  const int64_t t_lo = (int64_t)s * a.split_tokens;
  const int64_t t_hi = min(T, t_lo + (int64_t)a.split_tokens);
  if (t_lo >= t_hi) return;
  const int m = a.rank, gq = a.group, Hq = a.num_q_heads, n = a.num_chunks;
  const int r = a.rope_dim, half = r >> 1;
  const int64_t F = (int64_t)a.heads * kD;
  const uint16_t* kb = (const uint16_t*)a.data[0] + (int64_t)l * a.layer_stride[0] +
                       (int64_t)g * a.head_stride[0] + 4 * c;
  const uint16_t* vb = (const uint16_t*)a.data[1] + (int64_t)l * a.layer_stride[1] +
                       (int64_t)g * a.head_stride[1] + 4 * c;
  const uint16_t* ukb = MU > 0 ? (const uint16_t*)a.U[0] + (int64_t)l * T * m : nullptr;
  const uint16_t* uvb = MU > 0 ? (const uint16_t*)a.U[1] + (int64_t)l * T * m : nullptr;
  const uint32_t ss0 = (uint32_t)a.slot_stride[0], ss1 = (uint32_t)a.slot_stride[1];
  const uint32_t ps0 = (uint32_t)a.page_stride[0], ps1 = (uint32_t)a.page_stride[1];
  const uint32_t P = (uint32_t)a.page_size;
  const int psh = (P != 0u && (P & (P - 1u)) == 0u) ? __builtin_ctz(P) : -1;

  for (int64_t t0 = t_lo; t0 < t_hi;) {
    const int j = chunk_at(a.offsets, n, t0);
    const int64_t s1 = min(t_hi, a.offsets[j + 1]);
    if (s1 <= t0) break;  // offsets that do not cover the range: nothing more here

    // ---- segment set-up: rotated query and V_K^T q of each query head
    for (int idx = tid; idx < G * kD; idx += kThreads) {
      const int h = idx / kD, d = idx - h * kD;
      float v = 0.f;
      if (h < gq) {
        const float* qh = a.q + ((int64_t)l * Hq + g * gq + h) * kD;
        v = qh[d];
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
            const float b = qh[dp];
            v = first ? fmaf(v, cs.x, -(b * cs.y)) : fmaf(v, cs.x, b * cs.y);
          }
        }
      }
      sq[h][d] = v * a.scale_log2;
    }
    if constexpr (MU > 0) {
      for (int idx = tid; idx < G * m; idx += kThreads) {
        const int h = idx / m, k = idx - h * m;
        float w = 0.f;
        if (h < gq) {
          const float* qh = a.q + ((int64_t)l * Hq + g * gq + h) * kD;
          const uint16_t* vk =
              (const uint16_t*)a.V[0] + (((int64_t)l * n + j) * F + (int64_t)g * kD) * m + k;
          for (int d = 0; d < kD; ++d) w = fmaf(qh[d], bf16_at(vk + (int64_t)d * m), w);
        }
        sw[h][k] = w * a.scale_log2;
      }
    }
    __syncthreads();
    float qt[G][4], wk[G][MUX];
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 4; ++e) qt[h][e] = sq[h][4 * c + e];
#pragma unroll
      for (int k = 0; k < MUX; ++k) wk[h][k] = (MU > 0 && c * MU + k < m) ? sw[h][c * MU + k] : 0.f;
    }

    // ---- stream the segment's tokens: row group rg takes tokens t0 + rg + 8 b + ...
    float mr[G], lr[G], acc[G][4], ub[G][MUX];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mr[h] = -INFINITY;
      lr[h] = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[h][e] = 0.f;
#pragma unroll
      for (int k = 0; k < MUX; ++k) ub[h][k] = 0.f;
    }
    for (int64_t base = t0; base < s1; base += kRowGroups * NB) {
      u32x2_t kx[NB], vx[NB];
      float uk[NB][MUX], uv[NB][MUX];
      bool ok[NB];
      // Row offsets inside a layer fit in 32 bits (checked on the host); tokens < 2^30.
      const uint32_t t_first = (uint32_t)(base + rg);
      uint32_t ck = t_first * ss0, cv = t_first * ss1;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint32_t t = t_first + kRowGroups * b;
        ok[b] = (int64_t)t < s1;
        uint32_t sk = ck, sv = cv;
        ck += kRowGroups * ss0;
        cv += kRowGroups * ss1;
        if constexpr (PAGED) {
          sk = sv = 0u;
          if (ok[b]) {
            const uint32_t pi = psh >= 0 ? t >> psh : t / P, si = t - pi * P;
            const int32_t pg = a.block_table[pi];
            ok[b] = pg >= 0 && pg < a.num_pages;
            sk = (uint32_t)pg * ps0 + si * ss0;
            sv = (uint32_t)pg * ps1 + si * ss1;
          }
        }
        kx[b] = u32x2_t{0u, 0u};
        vx[b] = u32x2_t{0u, 0u};
        if (ok[b]) {
          kx[b] = __builtin_nontemporal_load((const u32x2_t*)(kb + sk));
          vx[b] = __builtin_nontemporal_load((const u32x2_t*)(vb + sv));
        }
#pragma unroll
        for (int k = 0; k < MUX; ++k) {
          const bool uon = MU > 0 && ok[b] && c * MU + k < m;
          uk[b][k] = uon ? bf16_at(ukb + (int64_t)t * m + c * MU + k) : 0.f;
          uv[b][k] = uon ? bf16_at(uvb + (int64_t)t * m + c * MU + k) : 0.f;
        }
      }
      float sc[NB][G];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float k0 = bf16_lo(kx[b].x), k1 = bf16_hi(kx[b].x);
        const float k2 = bf16_lo(kx[b].y), k3 = bf16_hi(kx[b].y);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float p = qt[h][0] * k0;
          p = fmaf(qt[h][1], k1, p);
          p = fmaf(qt[h][2], k2, p);
          p = fmaf(qt[h][3], k3, p);
#pragma unroll
          for (int k = 0; k < MUX; ++k) p = fmaf(wk[h][k], uk[b][k], p);
          p = sum32(p);
          sc[b][h] = ok[b] ? p : -INFINITY;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mb = sc[0][h];
#pragma unroll
        for (int b = 1; b < NB; ++b) mb = fmaxf(mb, sc[b][h]);
        const float mn = fmaxf(mr[h], mb);
        const float corr = weight(mr[h], mn);
        lr[h] *= corr;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[h][e] *= corr;
#pragma unroll
        for (int k = 0; k < MUX; ++k) ub[h][k] *= corr;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float p = weight(sc[b][h], mn);
          lr[h] += p;
          acc[h][0] = fmaf(p, bf16_lo(vx[b].x), acc[h][0]);
          acc[h][1] = fmaf(p, bf16_hi(vx[b].x), acc[h][1]);
          acc[h][2] = fmaf(p, bf16_lo(vx[b].y), acc[h][2]);
          acc[h][3] = fmaf(p, bf16_hi(vx[b].y), acc[h][3]);
#pragma unroll
          for (int k = 0; k < MUX; ++k) ub[h][k] = fmaf(p, uv[b][k], ub[h][k]);
        }
        mr[h] = mn;
      }
    }

    // ---- merge: the two row groups of a wave, then the four waves
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(mr[h], 32);
      const float M = fmaxf(mr[h], mo);
      const float fs = weight(mr[h], M), fo = weight(mo, M);
      lr[h] = lr[h] * fs + __shfl_xor(lr[h], 32) * fo;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[h][e] = acc[h][e] * fs + __shfl_xor(acc[h][e], 32) * fo;
#pragma unroll
      for (int k = 0; k < MUX; ++k) ub[h][k] = ub[h][k] * fs + __shfl_xor(ub[h][k], 32) * fo;
      mr[h] = M;
    }
    if (lane < 32) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (c == 0) {
          sred[wave][h][0] = mr[h];
          sred[wave][h][1] = lr[h];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sred[wave][h][2 + 4 * c + e] = acc[h][e];
#pragma unroll
        for (int k = 0; k < MUX; ++k)
          if (MU > 0 && c * MU + k < m) sred[wave][h][2 + kD + c * MU + k] = ub[h][k];
      }
    }
    __syncthreads();
    if constexpr (MU > 0) {
      for (int idx = tid; idx < G * m; idx += kThreads) {
        const int h = idx / m, k = idx - h * m;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sred[w][h][0]);
        float u = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) u = fmaf(weight(sred[w][h][0], M), sred[w][h][2 + kD + k], u);
        sub[h][k] = u;
      }
      __syncthreads();
    }
    for (int idx = tid; idx < G * kD; idx += kThreads) {
      const int h = idx / kD, d = idx - h * kD;
      if (h >= gq) continue;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sred[w][h][0]);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = weight(sred[w][h][0], M);
        L = fmaf(f, sred[w][h][1], L);
        A = fmaf(f, sred[w][h][2 + d], A);
      }
      if constexpr (MU > 0) {
        const uint16_t* vv =
            (const uint16_t*)a.V[1] + (((int64_t)l * n + j) * F + (int64_t)g * kD + d) * m;
        for (int k = 0; k < m; ++k) A = fmaf(bf16_at(vv + k), sub[h][k], A);
      }
      float* slot = a.ws + (((int64_t)l * Hq + g * gq + h) * a.slots + (s + j)) * kAttendPartial;
      if (d == 0) {
        slot[0] = M;
        slot[1] = L;
      }
      slot[2 + d] = A;
    }
    __syncthreads();  // the next segment restages the shared arrays
    t0 = s1;
  }
}

// One workgroup per (layer, query head), thread d: merges the partial slots the split
// kernel wrote, walking the same (split, chunk) segments.
__global__ __launch_bounds__(kD) void attend_combine(AttendArgs a) {
  const int Hq = a.num_q_heads;
  const int hq = (int)(blockIdx.x % (uint32_t)Hq);
  const int l = (int)(blockIdx.x / (uint32_t)Hq);
  const int d = threadIdx.x;
  const float* base = a.ws + ((int64_t)l * Hq + hq) * a.slots * kAttendPartial;
  const int64_t T = a.total_tokens;
  float M = -INFINITY;
  for (int pass = 0; pass < 2; ++pass) {
    float num = 0.f, den = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const int64_t t_lo = (int64_t)s * a.split_tokens;
      const int64_t t_hi = min(T, t_lo + (int64_t)a.split_tokens);
      for (int64_t t0 = t_lo; t0 < t_hi;) {
        const int j = chunk_at(a.offsets, a.num_chunks, t0);
        const int64_t s1 = min(t_hi, a.offsets[j + 1]);
        if (s1 <= t0) break;
        const float* slot = base + (int64_t)(s + j) * kAttendPartial;
        const float ls = slot[1];
        if (ls > 0.f) {
          if (pass == 0) {
            M = fmaxf(M, slot[0]);
          } else {
            const float f = exp2f(slot[0] - M);
            den = fmaf(f, ls, den);
            num = fmaf(f, slot[2 + d], num);
          }
        }
        t0 = s1;
      }
    }
    if (pass == 1) {
      const int64_t o = (int64_t)l * Hq + hq;
      a.out[o * kD + d] = den > 0.f ? num / den : 0.f;
      if (a.lse != nullptr && d == 0)
        a.lse[o] = den > 0.f ? (M + log2f(den)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  const dim3 grid1((unsigned)((int64_t)a.num_layers * a.heads * a.splits));
  const int mu = (a.rank + 31) / 32;
  const int G = a.group <= 2 ? 2 : a.group <= 4 ? 4 : 8;
#define KAMERA_ATT(GG, MM, PG)                                                                 \
  hipLaunchKernelGGL((attend_split<GG, MM, (GG >= 8 ? 2 : 4), PG>), grid1, dim3(kThreads), 0, s, a)
#define KAMERA_ATT_MU(GG, PG)                          \
  do {                                                 \
    if (mu == 0) KAMERA_ATT(GG, 0, PG);                \
    else if (mu == 1) KAMERA_ATT(GG, 1, PG);           \
    else if (mu == 2) KAMERA_ATT(GG, 2, PG);           \
    else KAMERA_ATT(GG, 4, PG);                        \
  } while (0)
#define KAMERA_ATT_G(PG)                               \
  do {                                                 \
    if (G == 2) KAMERA_ATT_MU(2, PG);                  \
    else if (G == 4) KAMERA_ATT_MU(4, PG);             \
    else KAMERA_ATT_MU(8, PG);                         \
  } while (0)
  if (a.splits > 0) {  // no tokens: only the merge runs, writing 0 and -inf
    if (a.page_size > 0) KAMERA_ATT_G(true);
    else KAMERA_ATT_G(false);
  }
#undef KAMERA_ATT_G
#undef KAMERA_ATT_MU
#undef KAMERA_ATT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid2((unsigned)((int64_t)a.num_layers * a.num_q_heads));
  hipLaunchKernelGGL(attend_combine, grid2, dim3(kD), 0, s, a);
  return hipGetLastError();
}

}  // namespace kamera
