// gfx950 kernels of the Kamera relocate + patch operator.
//
// Operator ("Kamera: KV Cache Multimodal Unificado e Invariante a Posicao para Reuso
// sem Treinamento", gist.science/pt/paper/2606.23581, §2, reuse equation):
//     out = round( R(delta_j) x + U_m V_m^T )
// applied in place to every layer, channel and chunk of a KV cache.  R(delta) turns
// each NeoX pair (i, i + r/2) of a head by angle delta * theta^(-2i/r) (§2,
// "Relocacao"); the rank-m patch adds sum_k U[t][k] * V[f][k] to element (t, f) (§2,
// "Aplicacao de Patch").
//
// Three kernels:
//   rotate_bf16            m = 0: only the rotated dims of rotating channels are read and
//                          written (§3, sliding-window survival: no patch is needed).
//   relocate_patch_mfma    m > 0: rotation fused with the patch in one HBM pass; the
//                          patch is a [16 x m] x [m x 16] product per tile on MFMA.
//   generic_rows           any shape, bf16 or fp32: one thread per (layer, token, head).
//
// Memory: each KV element is read once and written once, in place.  A wavefront owns
// whole 128-byte lines of the rows it writes.  Angles are formed in fp64 (delta up to
// 2^53 times a frequency near 1 needs fp64 to keep the phase error far below fp32
// rounding) and rounded to fp32 once per chunk; all element arithmetic is fp32.
#include <hip/hip_runtime.h>

#include "kamera_internal.h"

namespace kamera {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = 64 * kWavesPerBlock;

// ------------------------------------------------------------------ element helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4& v, float (&x)[8]) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// Two fp32 -> two bf16 with round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint4 pack8(const float (&y)[8]) {
  return make_uint4(pack2(y[0], y[1]), pack2(y[2], y[3]), pack2(y[4], y[5]), pack2(y[6], y[7]));
}

__device__ __forceinline__ float load_f(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ float load_f(const float* p) { return *p; }
__device__ __forceinline__ void store_f(uint16_t* p, float y) {
  *p = __builtin_bit_cast(uint16_t, static_cast<__bf16>(y));
}
__device__ __forceinline__ void store_f(float* p, float y) { *p = y; }

// ------------------------------------------------------------------ index helpers

// Chunk that owns token t: the last j with offsets[j] <= t (offsets[0] == 0 <= t).
__device__ __forceinline__ int find_chunk(const int64_t* off, int n, int64_t t) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Element offset of logical token t's slot inside one layer.  Paged: the block table
// maps logical page t / P to a pool page; a page id outside [0, num_pages) leaves
// the row untouched (ok = false) instead of touching memory outside the pool.
__device__ __forceinline__ int64_t slot_offset(const ChanArgs& ch, const CommonArgs& cm,
                                               int64_t t, bool& ok) {
  if (cm.page_size > 0) {
    const int tt = (int)t;
    const int64_t pg = cm.block_table[tt / cm.page_size];
    ok = pg >= 0 && pg < cm.num_pages;
    return pg * ch.page_stride + (int64_t)(tt % cm.page_size) * ch.slot_stride;
  }
  ok = true;
  return t * ch.slot_stride;
}

// cos and sin of delta * theta^(-2i/r): the angle is formed and reduced in fp64, then
// rounded to fp32.
__device__ __forceinline__ void phase(double theta, int r, int i, int64_t delta,
                                      float& c, float& s) {
  const double w = pow(theta, -2.0 * (double)i / (double)r);
  const double phi = (double)delta * w;
  double sd, cd;
  sincos(phi, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

// ------------------------------------------------------------------ rotation only

// One wavefront streams the rows (token, head) of `range_tokens` tokens of one layer.
// A row's rotated part is r = 16 * LPR dims: LPR lanes each own 8 dims of the first
// half and their 8 partners in the second half (two 16-byte loads, two 16-byte
// stores), so 64 / LPR rows move per wavefront step.  Dims >= r are never touched.
template <int LPR>
__global__ __launch_bounds__(kBlock) void rotate_bf16(ChanArgs ch, CommonArgs cm) {
  constexpr int HALF = 8 * LPR;
  constexpr int RPW = 64 / LPR;
  constexpr int NS = (HALF + 63) / 64;
  constexpr int UNR = 4;
  const int lane = threadIdx.x & 63;
  const int64_t unit = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (unit >= (int64_t)cm.num_layers * cm.nranges) return;
  const int64_t layer = unit / cm.nranges;
  int64_t t0 = (unit - layer * cm.nranges) * cm.range_tokens;
  const int64_t t1 = min(t0 + (int64_t)cm.range_tokens, cm.total_tokens);
  const int q = lane % LPR;
  const int rho = lane / LPR;
  const int H = ch.heads;
  uint16_t* base = (uint16_t*)ch.data + layer * ch.layer_stride;
  int j = find_chunk(cm.offsets, cm.num_chunks, t0);
  while (t0 < t1 && j < cm.num_chunks) {
    const int64_t seg_end = min(t1, cm.offsets[j + 1]);
    const int64_t dj = cm.delta[j];
    if (seg_end > t0 && dj != 0) {
      // Lane l forms pair frequency l (and l + 64); lanes then gather their 8.
      float cown[NS], sown[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int i = lane + 64 * s;
        cown[s] = 1.f;
        sown[s] = 0.f;
        if (i < HALF) phase(cm.theta, 2 * HALF, i, dj, cown[s], sown[s]);
      }
      float cs[8], sn[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * q + e;
        float c = __shfl(cown[0], i & 63);
        float s = __shfl(sown[0], i & 63);
#pragma unroll
        for (int k = 1; k < NS; ++k) {
          const float c1 = __shfl(cown[k], i & 63);
          const float s1 = __shfl(sown[k], i & 63);
          if ((i >> 6) == k) { c = c1; s = s1; }
        }
        cs[e] = c;
        sn[e] = s;
      }
      const int nrows = (int)(seg_end - t0) * H;
      for (int r0 = 0; r0 < nrows; r0 += RPW * UNR) {
        uint4 va[UNR], vb[UNR];
        uint16_t* rowp[UNR];
        bool ok[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int R = r0 + u * RPW + rho;
          ok[u] = R < nrows;
          rowp[u] = base;
          if (ok[u]) {
            const int tl = R / H;
            const int h = R - tl * H;
            bool pok;
            const int64_t so = slot_offset(ch, cm, t0 + tl, pok);
            ok[u] = pok;
            rowp[u] = base + so + (int64_t)h * ch.head_stride + 8 * q;
          }
          if (ok[u]) {
            va[u] = *(const uint4*)rowp[u];
            vb[u] = *(const uint4*)(rowp[u] + HALF);
          }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          if (!ok[u]) continue;
          float a[8], b[8];
          unpack8(va[u], a);
          unpack8(vb[u], b);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float an = fmaf(a[e], cs[e], -(b[e] * sn[e]));
            const float bn = fmaf(b[e], cs[e], a[e] * sn[e]);
            a[e] = an;
            b[e] = bn;
          }
          *(uint4*)rowp[u] = pack8(a);
          *(uint4*)(rowp[u] + HALF) = pack8(b);
        }
      }
    }
    t0 = max(t0, seg_end);
    ++j;
  }
}

// ------------------------------------------------------------------ rotation + patch (MFMA)

// Patch fragment of 8 consecutive k (bf16): a 16-byte load when all 8 lie below m and
// rows are 16-byte aligned (m % 8 == 0), else element loads with zero fill.
__device__ __forceinline__ bf16x8_t load_frag(const uint16_t* row, int k0, int m, bool m8) {
  if (m8 && k0 + 8 <= m) return __builtin_bit_cast(bf16x8_t, *(const uint4*)(row + k0));
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (k0 + e < m) ? row[k0 + e] : (uint16_t)0;
  uint4 w = make_uint4(v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                       v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16));
  return __builtin_bit_cast(bf16x8_t, w);
}

// Work unit of one wavefront: NT "tasks" of one channel and layer, over `range_tokens`
// tokens, 16 tokens per step.  A task is 64 features of one head, kept as two 32-wide
// slabs: a rotating pair task holds dims [32i, 32i+32) and their partners
// [r/2 + 32i, r/2 + 32i + 32); a plain task holds dims [r + 64i', r + 64i' + 64).
//
// Lane l works on token (l & 15) of the step and on dims 8g..8g+7 (g = l >> 4) of each
// slab: a NeoX pair never leaves the lane.  The patch of one slab is two MFMA
// 16x16x32 bf16 tiles per 32 k:  D[f][t] = C[f][t] + sum_k V[f][k] U[t][k], with
// A = V rows (features), B = U rows (tokens).  The MFMA output layout gives lane l
// rows 4g..4g+3 of column l & 15; the A rows are ordered so that output row 4g+i of
// tile p is feature 8g + 4p + i of the slab.  The lane's own rotated values are thus
// the C operand, and the output lands in the lane that stores it.
template <int NT, int MK>
__global__ __launch_bounds__(kBlock) void relocate_patch_mfma(ChanArgs ch0, ChanArgs ch1,
                                                              CommonArgs cm,
                                                              int64_t units_per_layer) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int64_t unit = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (unit >= (int64_t)cm.num_layers * units_per_layer) return;
  const int64_t layer = unit / units_per_layer;
  int64_t rem = unit - layer * units_per_layer;
  const bool second = rem >= ch0.units;
  if (second) rem -= ch0.units;
  const ChanArgs ch = second ? ch1 : ch0;
  const int64_t range = rem / ch.groups;
  const int group = (int)(rem - range * ch.groups);

  const int m = cm.rank;
  const bool m8 = (m & 7) == 0;
  const int F = ch.heads * ch.dim;
  const int r = ch.rope_dim;
  const int npair = r >> 6;
  const int ntask = ch.heads * ch.tasks_per_head;

  bool tv[NT], tp[NT];
  int ti[NT], dd[NT][2], fb[NT][2];
  int64_t hoff[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    const int tau = group * NT + k;
    tv[k] = tau < ntask;
    const int h = tau / ch.tasks_per_head;
    const int i = tau - h * ch.tasks_per_head;
    tp[k] = i < npair;
    ti[k] = i;
    dd[k][0] = tp[k] ? 32 * i : r + 64 * (i - npair);
    dd[k][1] = tp[k] ? (r >> 1) + 32 * i : dd[k][0] + 32;
    fb[k][0] = h * ch.dim + dd[k][0];
    fb[k][1] = h * ch.dim + dd[k][1];
    hoff[k] = (int64_t)h * ch.head_stride;
  }

  const uint16_t* Ul = (const uint16_t*)ch.U + layer * cm.total_tokens * m;
  const uint16_t* Vl = (const uint16_t*)ch.V + layer * (int64_t)cm.num_chunks * F * m;
  uint16_t* base = (uint16_t*)ch.data + layer * ch.layer_stride;

  int64_t t0 = range * cm.range_tokens;
  const int64_t t1 = min(t0 + (int64_t)cm.range_tokens, cm.total_tokens);
  int j = find_chunk(cm.offsets, cm.num_chunks, t0);
  while (t0 < t1 && j < cm.num_chunks) {
    const int64_t seg_end = min(t1, cm.offsets[j + 1]);
    if (seg_end > t0) {
      const int64_t dj = cm.delta[j];
      // Feature factor of chunk j, resident in registers for the whole segment.
      const uint16_t* Vj = Vl + (int64_t)j * F * m;
      bf16x8_t vf[NT][2][2][MK];
#pragma unroll
      for (int k = 0; k < NT; ++k)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int ks = 0; ks < MK; ++ks) {
              const int f = fb[k][s] + 8 * (col >> 2) + 4 * p + (col & 3);
              vf[k][s][p][ks] = tv[k] ? load_frag(Vj + (int64_t)f * m, 32 * ks + 8 * g, m, m8)
                                      : load_frag(Vj, 0, 0, m8);
            }
      // Phase of the lane's 8 pairs per rotating task.
      float cs[NT][8], sn[NT][8];
      const bool rot = dj != 0;
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        float c = 1.f, s = 0.f;
        if (rot && tv[k] && tp[k]) phase(cm.theta, r, 32 * ti[k] + (lane & 31), dj, c, s);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          cs[k][e] = __shfl(c, 8 * g + e);
          sn[k][e] = __shfl(s, 8 * g + e);
        }
      }

      uint4 xc[NT][2], xn[NT][2];
      bf16x8_t uc[MK], un[MK];
      uint16_t* rc[NT];
      uint16_t* rn[NT];
      bool okc, okn;
      auto load_tile = [&](int64_t ts, uint4 (&xv)[NT][2], bf16x8_t (&uf)[MK],
                           uint16_t* (&rp)[NT], bool& ok) {
        const int64_t tok = ts + col;
        ok = tok < seg_end;
        int64_t so = 0;
        if (ok) {
          bool pok;
          so = slot_offset(ch, cm, tok, pok);
          ok = pok;
        }
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          rp[k] = base + so + hoff[k];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            xv[k][s] = make_uint4(0, 0, 0, 0);
            if (ok && tv[k]) xv[k][s] = *(const uint4*)(rp[k] + dd[k][s] + 8 * g);
          }
        }
        const uint16_t* urow = Ul + (ok ? tok : 0) * m;
#pragma unroll
        for (int ks = 0; ks < MK; ++ks) {
          uf[ks] = load_frag(urow, 0, 0, m8);
          if (ok) uf[ks] = load_frag(urow, 32 * ks + 8 * g, m, m8);
        }
      };

      load_tile(t0, xc, uc, rc, okc);
      for (int64_t ts = t0; ts < seg_end; ts += 16) {
        const bool more = ts + 16 < seg_end;
        if (more) load_tile(ts + 16, xn, un, rn, okn);

        f32x4_t acc[NT][2][2];
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          float a[8], b[8];
          unpack8(xc[k][0], a);
          unpack8(xc[k][1], b);
          if (rot && tp[k]) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float an = fmaf(a[e], cs[k][e], -(b[e] * sn[k][e]));
              const float bn = fmaf(b[e], cs[k][e], a[e] * sn[k][e]);
              a[e] = an;
              b[e] = bn;
            }
          }
          acc[k][0][0] = f32x4_t{a[0], a[1], a[2], a[3]};
          acc[k][0][1] = f32x4_t{a[4], a[5], a[6], a[7]};
          acc[k][1][0] = f32x4_t{b[0], b[1], b[2], b[3]};
          acc[k][1][1] = f32x4_t{b[4], b[5], b[6], b[7]};
        }
#pragma unroll
        for (int ks = 0; ks < MK; ++ks)
#pragma unroll
          for (int k = 0; k < NT; ++k)
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
              for (int p = 0; p < 2; ++p)
                acc[k][s][p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[k][s][p][ks], uc[ks],
                                                                       acc[k][s][p], 0, 0, 0);
        if (okc) {
#pragma unroll
          for (int k = 0; k < NT; ++k) {
            if (!tv[k]) continue;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              float y[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) y[e] = acc[k][s][e >> 2][e & 3];
              *(uint4*)(rc[k] + dd[k][s] + 8 * g) = pack8(y);
            }
          }
        }
        if (more) {
#pragma unroll
          for (int k = 0; k < NT; ++k) {
            xc[k][0] = xn[k][0];
            xc[k][1] = xn[k][1];
            rc[k] = rn[k];
          }
#pragma unroll
          for (int ks = 0; ks < MK; ++ks) uc[ks] = un[ks];
          okc = okn;
        }
      }
    }
    t0 = max(t0, seg_end);
    ++j;
  }
}

// ------------------------------------------------------------------ generic rows

template <typename T>
__device__ __forceinline__ float dot_patch(const T* u, const T* v, int m) {
  float s = 0.f;
  for (int k = 0; k < m; ++k) s = fmaf(load_f(u + k), load_f(v + k), s);
  return s;
}

// One thread per (layer, token, head) row; any dim, any even rope_dim, any rank.
template <typename T>
__global__ __launch_bounds__(kBlock) void generic_rows(ChanArgs ch, CommonArgs cm) {
  const int64_t H = ch.heads, Tt = cm.total_tokens;
  const int64_t nrows = (int64_t)cm.num_layers * Tt * H;
  const int m = cm.rank, D = ch.dim, r = ch.rope_dim, half = r >> 1;
  const int64_t F = H * D;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nrows;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t h = idx % H;
    const int64_t rest = idx / H;
    const int64_t t = rest % Tt;
    const int64_t layer = rest / Tt;
    const int j = find_chunk(cm.offsets, cm.num_chunks, t);
    const int64_t dj = cm.delta[j];
    if (m == 0 && (dj == 0 || r == 0)) continue;
    bool ok = true;
    int64_t so;
    if (cm.page_size > 0) {
      const int64_t pg = cm.block_table[t / cm.page_size];
      ok = pg >= 0 && pg < cm.num_pages;
      so = pg * ch.page_stride + (t % cm.page_size) * ch.slot_stride;
    } else {
      so = t * ch.slot_stride;
    }
    if (!ok) continue;
    T* row = (T*)ch.data + layer * ch.layer_stride + so + h * ch.head_stride;
    const T* u = (const T*)ch.U + (layer * Tt + t) * m;
    const T* vr = (const T*)ch.V + ((layer * cm.num_chunks + j) * F + h * D) * m;
    for (int i = 0; i < half; ++i) {
      float a = load_f(row + i), b = load_f(row + i + half);
      if (dj != 0) {
        float c, s;
        phase(cm.theta, r, i, dj, c, s);
        const float an = fmaf(a, c, -(b * s));
        const float bn = fmaf(b, c, a * s);
        a = an;
        b = bn;
      }
      if (m > 0) {
        a += dot_patch(u, vr + (int64_t)i * m, m);
        b += dot_patch(u, vr + (int64_t)(i + half) * m, m);
      }
      store_f(row + i, a);
      store_f(row + i + half, b);
    }
    if (m > 0)
      for (int d = r; d < D; ++d) store_f(row + d, load_f(row + d) + dot_patch(u, vr + (int64_t)d * m, m));
  }
}

}  // namespace

// ------------------------------------------------------------------ launchers

hipError_t launch_rotate_bf16(const ChanArgs& ch, const CommonArgs& cm, hipStream_t s) {
  const int64_t units = (int64_t)cm.num_layers * cm.nranges;
  const dim3 grid((unsigned)((units + kWavesPerBlock - 1) / kWavesPerBlock));
  switch (ch.rope_dim / 16) {
    case 1: hipLaunchKernelGGL(rotate_bf16<1>, grid, dim3(kBlock), 0, s, ch, cm); break;
    case 2: hipLaunchKernelGGL(rotate_bf16<2>, grid, dim3(kBlock), 0, s, ch, cm); break;
    case 4: hipLaunchKernelGGL(rotate_bf16<4>, grid, dim3(kBlock), 0, s, ch, cm); break;
    case 8: hipLaunchKernelGGL(rotate_bf16<8>, grid, dim3(kBlock), 0, s, ch, cm); break;
    case 16: hipLaunchKernelGGL(rotate_bf16<16>, grid, dim3(kBlock), 0, s, ch, cm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_relocate_patch_mfma(const ChanArgs* ch, int nch, const CommonArgs& cm,
                                      int tasks_per_wave, hipStream_t s) {
  ChanArgs c0 = ch[0];
  ChanArgs c1 = nch > 1 ? ch[1] : ch[0];
  if (nch == 1) c1.units = 0;
  const int64_t upl = c0.units + c1.units;
  const int64_t units = (int64_t)cm.num_layers * upl;
  const dim3 grid((unsigned)((units + kWavesPerBlock - 1) / kWavesPerBlock));
  const int mk = (cm.rank + 31) / 32;
  if (tasks_per_wave != 1) return hipErrorInvalidValue;
  if (mk == 1)
    hipLaunchKernelGGL((relocate_patch_mfma<1, 1>), grid, dim3(kBlock), 0, s, c0, c1, cm, upl);
  else if (mk == 2)
    hipLaunchKernelGGL((relocate_patch_mfma<1, 2>), grid, dim3(kBlock), 0, s, c0, c1, cm, upl);
  else if (mk <= 4)
    hipLaunchKernelGGL((relocate_patch_mfma<1, 4>), grid, dim3(kBlock), 0, s, c0, c1, cm, upl);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_generic(const ChanArgs& ch, const CommonArgs& cm, int dtype, hipStream_t s) {
  const int64_t nrows = (int64_t)cm.num_layers * cm.total_tokens * ch.heads;
  int64_t blocks = (nrows + kBlock - 1) / kBlock;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (dtype == 0)
    hipLaunchKernelGGL(generic_rows<uint16_t>, dim3((unsigned)blocks), dim3(kBlock), 0, s, ch, cm);
  else
    hipLaunchKernelGGL(generic_rows<float>, dim3((unsigned)blocks), dim3(kBlock), 0, s, ch, cm);
  return hipGetLastError();
}

}  // namespace kamera
