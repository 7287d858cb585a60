// gfx950 kernels of the Kamera relocate + patch operator.
//
// Operator ("Kamera: KV Cache Multimodal Unificado e Invariante a Posicao para Reuso
// sem Treinamento", gist.science/pt/paper/2606.23581, §2, reuse equation):
//     out = round( R(delta_j) x + U_m V_m^T )
// for every layer, channel and chunk of a KV cache, in place or (recall) from a
// source cache into a destination cache.  R(delta) turns each rotary pair of a head
// by angle delta * theta^(-2i/r) (§2, "Relocacao"): NeoX half-split pairs
// (i, i + r/2) or interleaved pairs (2i, 2i + 1), and with M-RoPE sections each pair
// takes the delta of its section.  The rank-m patch adds sum_k U[t][k] * V[f][k] to
// element (t, f) (§2, "Aplicacao de Patch").
//
// Kernels:
//   table_inverse_*      pool page -> logical page, into the caller's workspace (pool order)
//   rotate_rows          m = 0 in place: only the rotated dims of rotating channels
//                        are read and written (§3, sliding-window survival: no patch
//                        is needed).
//   relocate_patch_rows  m > 0, or any recall: rotation fused with the patch in one
//                        HBM pass; the patch of a 16-token x 128-feature tile is 8
//                        MFMA 16x16x32 bf16 tiles per 32 k.  The head launch covers
//                        each token group up to the end of its first chunk, and in
//                        place, with no more chunk boundaries than groups, one unit
//                        per boundary covers each further chunk's part of a cut group;
//                        otherwise a tail launch (TAIL) covers the rest of the cut
//                        groups.  OUT writes a destination cache.
//                        Its VALU form (a measurement variant) sums the patch with
//                        v_dot2_f32_bf16 instead.
//   generic_rows         any shape, bf16 or fp32: one thread per (layer, token, head).
//
// Memory shape of the tuned kernels (what streams well on MI355X HBM3E): every KV load
// and store is a 16-byte (fp8: 8-byte) nontemporal buffer access through a resource
// over the current layer, with 32-bit byte offsets; a row a lane skips takes an offset
// past the range, which the hardware turns into a zero load and a dropped store, so no
// memory access sits behind a branch.  16 consecutive lanes cover one 256-byte row of
// 128 features (or LPR lanes cover the rotated part of a row), so each wave
// instruction touches whole 128-byte lines; a wavefront handles one to four 16-token
// tiles and exits, and consecutive workgroups sweep one compact address range
// together (the numbering keeps a token group's feature blocks on one XCD).  Per-chunk
// state (phases, feature factor V) is built once per workgroup in LDS.  Angles:
// delta * omega_i is formed in fp64 with omega_i from the host, reduced by pi/2 in
// fp64, and its cos and sin are rounded to fp32; all element arithmetic is fp32 with
// one rounding to bf16 at the end.
//
// Keeping HBM busy is a matter of bytes in flight per CU.  A launch over one chunk
// therefore (a) reads its uniform state (chunk end and delta, pool pages) with scalar
// loads before anything else, (b) requests the chunk's feature factor straight into LDS
// (no registers, no wait behind row data), and (c) has each wave request its first two
// 16-token tiles together (NT = 2: two tiles in flight per wave at three waves per SIMD).
// A paged cache with a caller workspace is swept in pool order (POOL): workgroups cover
// consecutive pool slots, the inverse block table gives each tile's logical page, and
// the tile's rows are requested before that lookup returns.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "kamera_internal.h"
#include "rope_device.h"

namespace kamera {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = 64 * kWavesPerBlock;

// ------------------------------------------------------------------ element helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const u32x4_t& v, float (&x)[8]) {
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

__device__ __forceinline__ u32x4_t pack8(const float (&y)[8]) {
  u32x4_t r;
  r.x = pack2(y[0], y[1]);
  r.y = pack2(y[2], y[3]);
  r.z = pack2(y[4], y[5]);
  r.w = pack2(y[6], y[7]);
  return r;
}


// Buffer addressing (gfx9 raw buffer: stride 0, dword data format in word 3).  A
// resource covers `bytes` bytes from a wave-uniform base; every access is range checked
// by the hardware, so a load at byte offset kOob reads zeros and a store there is
// dropped: rows a lane must skip take that offset instead of a branch.  aux = 2 sets
// the nontemporal bit.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// An offset chosen by a condition (row or kOob) reaches the access through an empty asm
// operand: otherwise the compiler may split the access into branches on that condition,
// and a load behind such a branch made it wait for every earlier load.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ void bload_nt(rsrc_t r, uint32_t off, u32x4_t& v) {
  v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)opaque(off), 0, 2);
}
__device__ __forceinline__ void bload_nt(rsrc_t r, uint32_t off, u32x2_t& v) {
  v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)opaque(off), 0, 2);
}
__device__ __forceinline__ void bstore_nt(rsrc_t r, uint32_t off, const u32x4_t& v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)opaque(off), 0, 2);
}
__device__ __forceinline__ void bstore_nt(rsrc_t r, uint32_t off, const u32x2_t& v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)opaque(off), 0, 2);
}
// 16 bytes at `off` through a resource, cached (factor rows are re-read by other waves).
__device__ __forceinline__ u32x4_t bload(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)opaque(off), 0, 0);
}

__device__ __forceinline__ float load_f(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ float load_f(const float* p) { return *p; }
__device__ __forceinline__ void store_f(uint16_t* p, float y) {
  *p = __builtin_bit_cast(uint16_t, static_cast<__bf16>(y));
}
__device__ __forceinline__ void store_f(float* p, float y) { *p = y; }

// ------------------------------------------------------------------ fp8 (OCP E4M3)
//
// 8-bit KV elements are OCP FP8 E4M3 codes (the format gfx950's conversions use): a
// lane's 8 elements are 8 bytes.  Code values become fp32 exactly; results go back
// rounded to the nearest code, ties to the even one.  The conversion turns magnitudes
// past the rounding range into NaN, so results are first clamped to +-448, the
// largest finite code (saturation), with the NaN-propagating maximum and minimum
// (v_maximum3_f32 / v_minimum3_f32): NaN passes the clamp unchanged.

// The two codes in the low (hi = false) or high 16 bits of w, as fp32.
__device__ __forceinline__ float2 fp8_pair(uint32_t w, bool hi) {
  const f32x2_t v = hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
                       : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  return make_float2(v.x, v.y);
}

__device__ __forceinline__ float sat_fp8(float y) {
  return __builtin_elementwise_minimum(__builtin_elementwise_maximum(y, -448.f), 448.f);
}

// `old` with its low (hi = false) or high 16 bits replaced by the codes of a and b.
__device__ __forceinline__ uint32_t fp8_put(float a, float b, uint32_t old, bool hi) {
  return hi ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat_fp8(a), sat_fp8(b), (int)old, true)
            : (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat_fp8(a), sat_fp8(b), (int)old, false);
}

__device__ __forceinline__ void unpack8(const u32x2_t& v, float (&x)[8]) {
  float2 p = fp8_pair(v.x, false);
  x[0] = p.x; x[1] = p.y;
  p = fp8_pair(v.x, true);
  x[2] = p.x; x[3] = p.y;
  p = fp8_pair(v.y, false);
  x[4] = p.x; x[5] = p.y;
  p = fp8_pair(v.y, true);
  x[6] = p.x; x[7] = p.y;
}

// Both halves of each word are written, so the first conversion's tied operand is
// seeded with the bits of its own first input (a register that dies there) rather
// than a zero that would need a move.
__device__ __forceinline__ u32x2_t pack8_fp8(const float (&y)[8]) {
  u32x2_t r;
  r.x = fp8_put(y[2], y[3], fp8_put(y[0], y[1], __float_as_uint(y[0]), false), true);
  r.y = fp8_put(y[6], y[7], fp8_put(y[4], y[5], __float_as_uint(y[4]), false), true);
  return r;
}


__device__ __forceinline__ float load_f(const uint8_t* p) { return fp8_pair(*p, false).x; }
__device__ __forceinline__ void store_f(uint8_t* p, float y) {
  *p = (uint8_t)(fp8_put(y, 0.f, 0u, false) & 0xffu);
}

template <int X>
__device__ __forceinline__ u32x4_t lane_xor4(const u32x4_t& v) {
  u32x4_t r;
  r.x = lane_xor<X>(v.x);
  r.y = lane_xor<X>(v.y);
  r.z = lane_xor<X>(v.z);
  r.w = lane_xor<X>(v.w);
  return r;
}

template <int X>
__device__ __forceinline__ u32x2_t lane_xor4(const u32x2_t& v) {
  u32x2_t r;
  r.x = lane_xor<X>(v.x);
  r.y = lane_xor<X>(v.y);
  return r;
}

// Word of results `y` with the halves flagged in `keep_lo` / `keep_hi` taken bit for
// bit from `x` (pairs whose section delta is 0 do not move).
__device__ __forceinline__ uint32_t keep_halves(uint32_t y, uint32_t x, bool keep_lo,
                                                bool keep_hi) {
  const uint32_t m = (keep_lo ? 0x0000ffffu : 0u) | (keep_hi ? 0xffff0000u : 0u);
  return (y & ~m) | (x & m);
}

// A lane's 8 results `o` with element e taken bit for bit from `x` where sn[e] == 0.
__device__ __forceinline__ u32x4_t keep_elems(u32x4_t o, const u32x4_t& x, const float (&sn)[8]) {
  o.x = keep_halves(o.x, x.x, sn[0] == 0.f, sn[1] == 0.f);
  o.y = keep_halves(o.y, x.y, sn[2] == 0.f, sn[3] == 0.f);
  o.z = keep_halves(o.z, x.z, sn[4] == 0.f, sn[5] == 0.f);
  o.w = keep_halves(o.w, x.w, sn[6] == 0.f, sn[7] == 0.f);
  return o;
}

__device__ __forceinline__ u32x2_t keep_elems(u32x2_t o, const u32x2_t& x, const float (&sn)[8]) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    uint32_t m = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) m |= sn[4 * w + b] == 0.f ? 0xffu << (8 * b) : 0u;
    o[w] = (o[w] & ~m) | (x[w] & m);
  }
  return o;
}

// Storage of the tuned kernels' elements: a lane holds 8 consecutive features of a
// row, bf16 in a u32x4 (feature pair p in word p) or fp8 in a u32x2 (feature pair p in
// half p & 1 of word p >> 1).  word / pair read feature pair pp; put and put_keep
// write it (put_keep takes the features flagged k0 / k1 bit for bit from the input
// words x).
template <bool Q>
struct Codec;

template <>
struct Codec<false> {
  using E = uint16_t;
  using XV = u32x4_t;
  static __device__ __forceinline__ uint32_t word(const XV& x, int pp) { return x[pp]; }
  static __device__ __forceinline__ float2 pair(uint32_t w, int) {
    return make_float2(bf16_lo(w), bf16_hi(w));
  }
  static __device__ __forceinline__ void put(XV& o, int pp, float y0, float y1) {
    o[pp] = pack2(y0, y1);
  }
  static __device__ __forceinline__ void put_keep(XV& o, const XV& x, int pp, float y0, float y1,
                                                  bool k0, bool k1) {
    o[pp] = keep_halves(pack2(y0, y1), x[pp], k0, k1);
  }
};

template <>
struct Codec<true> {
  using E = uint8_t;
  using XV = u32x2_t;
  static __device__ __forceinline__ uint32_t word(const XV& x, int pp) { return x[pp >> 1]; }
  static __device__ __forceinline__ float2 pair(uint32_t w, int pp) { return fp8_pair(w, pp & 1); }
  // The low half's conversion is seeded with y0's bits (the word is written whole).
  static __device__ __forceinline__ void put(XV& o, int pp, float y0, float y1) {
    const int k = pp >> 1;
    o[k] = fp8_put(y0, y1, (pp & 1) ? o[k] : __float_as_uint(y0), pp & 1);
  }
  static __device__ __forceinline__ void put_keep(XV& o, const XV& x, int pp, float y0, float y1,
                                                  bool k0, bool k1) {
    const int k = pp >> 1, sh = 16 * (pp & 1);
    const uint32_t m = (k0 ? 0xffu : 0u) | (k1 ? 0xff00u : 0u);
    const uint32_t v = (fp8_put(y0, y1, 0u, false) & 0xffffu & ~m) | ((x[k] >> sh) & m);
    o[k] = (pp & 1) ? ((o[k] & 0xffffu) | (v << 16)) : v;
  }
};

// ------------------------------------------------------------------ index helpers

// Chunk that owns token t: the last j with offsets[j] <= t (offsets[0] == 0 <= t), with
// its end offsets[j + 1] and its delta, in one round of loads: lane l reads
// offsets[base + l + 1] and delta[base + l], a ballot counts the chunks that start at
// or before t, and the owner's values come back by lane shuffle.  j lies in [0, n)
// whatever the offsets hold.  All lanes must call it.
struct ChunkRef {
  int j;
  int64_t end;
  int64_t delta;
};

// Whether chunk k moves at all: its delta, or any of its section deltas, is nonzero.
__device__ __forceinline__ int64_t chunk_moves(const CommonArgs& cm, int k) {
  if (cm.num_sections <= 1) return cm.delta[k];
  int64_t any = 0;
  for (int s = 0; s < cm.num_sections; ++s) any |= cm.delta[(int64_t)k * cm.num_sections + s];
  return any;
}

// The chunk holding token t, searched from chunk `from` on, by the whole wave: lane k
// reads the end and the motion of chunk base + k, a ballot counts the chunks that end
// at or before t.  ChunkRef::delta is nonzero iff the chunk moves (with sections it is
// not itself a delta: pair_delta gives those).
// SEC: 1 sections known present, 0 known absent, -1 decided at run time.
template <int SEC = -1>
__device__ __forceinline__ ChunkRef find_chunk_wave(const CommonArgs& cm, int64_t t,
                                                    int from = 0) {
  const int lane = threadIdx.x & 63;
  const int n = cm.num_chunks;
  const int64_t* off = cm.offsets;
  ChunkRef c{from, 0, 0};
  for (int base = from; base < n; base += 64) {
    const int k = base + lane;
    const int64_t e = k < n ? off[k + 1] : INT64_MAX;
    int64_t d = 0;
    if (k < n) d = SEC == 0 ? cm.delta[k] : chunk_moves(cm, k);
    const unsigned long long le = __ballot(e <= t);  // chunks that end at or before t
    const int cnt = __popcll(le);
    if (cnt < 64 || base + 64 >= n) {
      const int src = cnt < 64 ? cnt : 63;
      c.j = min(base + src, n - 1);
      c.end = __shfl(e, src);
      c.delta = __shfl(d, src);
      if (base + src >= n) {  // past the last chunk: clamp to it
        c.j = n - 1;
        c.end = off[n];
        c.delta = SEC == 0 ? cm.delta[n - 1] : chunk_moves(cm, n - 1);
      }
      break;
    }
  }
  return c;
}

// Section of rotary pair i (0 without M-RoPE).
__device__ __forceinline__ int section_of(const CommonArgs& cm, int i) {
  int s = 0;
#pragma unroll
  for (int k = 0; k < 3; ++k) s += (k + 1 < cm.num_sections && i >= cm.sec_end[k]) ? 1 : 0;
  return s;
}

// Delta that turns rotary pair i of chunk c.
__device__ __forceinline__ int64_t pair_delta(const CommonArgs& cm, const ChunkRef& c, int i) {
  if (cm.num_sections <= 1) return c.delta;
  return cm.delta[(int64_t)c.j * cm.num_sections + section_of(cm, i)];
}

// Chunk of token t for a single thread (generic kernel).
__device__ __forceinline__ int find_chunk(const int64_t* off, int n, int64_t t) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Generic-kernel phase: plain fp64 pow and sincos per element pair.
__device__ __forceinline__ void phase_generic(double theta, int r, int i, int64_t delta,
                                              float& c, float& s) {
  const double w = pow(theta, -2.0 * (double)i / (double)r);
  const double phi = (double)delta * w;
  double sd, cd;
  sincos(phi, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

// ------------------------------------------------------------------ rotation only

// Block-table entries a workgroup needs, staged once in LDS: pages [p0, p0 + n) cover
// tokens [tb0, t1).  Entries outside [0, num_pages) become -1 (their tokens are left
// untouched).  Returns p0.  The caller synchronises before reading `sbt`.
__device__ __forceinline__ int stage_table(const int32_t* table, int64_t num_pages, int P,
                                           int64_t tb0, int64_t t1, int* sbt) {
  // tuned kernels keep token ids below 2^30: 32-bit division
  const int p0 = (int)((uint32_t)tb0 / (uint32_t)P);
  const int n = (int)((uint32_t)(t1 - 1) / (uint32_t)P) + 1 - p0;
  for (int k = threadIdx.x; k < n; k += kBlock) {
    const int64_t pg = table[p0 + k];
    sbt[k] = (pg >= 0 && pg < num_pages) ? (int)pg : -1;
  }
  return p0;
}

__device__ __forceinline__ int stage_block_table(const CommonArgs& cm, int64_t tb0, int64_t t1,
                                                 int* sbt) {
  return stage_table(cm.block_table, cm.num_pages, cm.page_size, tb0, t1, sbt);
}

// Element offset, inside one layer, of the slot of token t (-1: token left untouched),
// in 32-bit arithmetic: the tuned kernels take channels whose per-layer extent is below
// 2^31 elements.  PAGED selects the addressing at compile time.
template <bool PAGED>
__device__ __forceinline__ int32_t slot32(int page_size, int page_shift, const int* sbt, int p0,
                                          int32_t page_stride, int32_t slot_stride, int t) {
  if constexpr (PAGED) {
    int pi, si;
    if (page_shift >= 0) {
      pi = t >> page_shift;
      si = t & (page_size - 1);
    } else {
      pi = t / page_size;
      si = t - pi * page_size;
    }
    const int pg = sbt[pi - p0];
    return pg < 0 ? -1 : pg * page_stride + si * slot_stride;
  } else {
    return t * slot_stride;
  }
}

// Workgroup = `block_tokens` tokens of one layer, every head, taken as rows (token,
// head) in order.  LPR lanes cover the rotated part of a row (8 dims each: 16 bytes of
// bf16, or 8 bytes of fp8 codes when Q; the rotation of code values needs no scale,
// which cancels); one wave
// instruction covers 64/LPR consecutive rows.  NeoX partner dims sit LPR/2 lanes away
// and arrive by a lane exchange; interleaved (IL) partners are the other half of the
// same 32-bit word.  Wave w takes row groups w, w + 4, ... (UNR of them per pass) and
// issues all their loads first.  Each wavefront then works on its own: it finds the
// chunks its rows belong to, forms that chunk's phases (one rotary pair per lane,
// gathered by lane shuffles) and finishes the rows.  Only a paged cache needs a
// workgroup barrier, once, for the staged block table.  Dims >= rope_dim are never
// touched; rows of chunks that do not move are not written; with M-RoPE sections, the
// dims of pairs whose section delta is 0 keep their bits.
//
// Row offsets inside a layer are 32-bit (the host checks the extent) and advance from
// one row group to the next by adds: the wave-uniform step of DR rows is dtl tokens and
// dh heads, with a carry when the head index wraps.
template <bool Q, int LPR, int UNR, bool PAGED, bool IL, bool SEC>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(UNR >= 4 ? 4 : 1)))
void rotate_rows(ChanArgs ch, CommonArgs cm) {
  using E = typename Codec<Q>::E;
  using XV = typename Codec<Q>::XV;
  constexpr int RPI = 64 / LPR;
  constexpr int HX = LPR / 2;
  constexpr int HALF = 4 * LPR;  // rotary pairs of a head: rope_dim / 2
  constexpr int ROWS = kWavesPerBlock * UNR * RPI;  // rows one pass of the block covers
  __shared__ int sbt[kMaxBlockTokens + 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t tgs = (uint32_t)cm.token_groups;  // grid = layers * tgs < 2^32
  const uint32_t layer = blockIdx.x / tgs;
  const uint32_t tg = blockIdx.x - layer * tgs;
  const int64_t tb0 = (int64_t)tg * cm.block_tokens;
  const int64_t t1 = min(tb0 + (int64_t)cm.block_tokens, cm.total_tokens);
  const int q = lane % LPR;
  const int rr = lane / LPR;
  // Rotary pair of each of the lane's 8 dims, and the sign of its partner term.
  const int fi0 = IL ? 4 * q : (q % HX) * 8;
  const float sgn = q < HX ? -1.f : 1.f;
  const int H = ch.heads;
  const int nrows = (int)(t1 - tb0) * H;
  // One layer through a buffer resource: rows the lane skips take byte offset kOob.
  const rsrc_t rkv = make_rsrc((E*)ch.data + (int64_t)layer * ch.layer_stride, ch.layer_bytes);
  // Offsets in uint32 arithmetic: every row the lane touches lies below 2^31, and rows
  // past the block's end (never loaded) may wrap harmlessly.
  const uint32_t ss = (uint32_t)ch.slot_stride, hs = (uint32_t)ch.head_stride;
  const int32_t ps = (int32_t)ch.page_stride;
  constexpr int DR = kWavesPerBlock * RPI;  // rows between a lane's row groups
  const int dtl = DR / H, dh = DR - dtl * H;
  const uint32_t dstep = (uint32_t)dtl * ss + (uint32_t)dh * hs;  // contiguous offset step
  const uint32_t carry = ss - (uint32_t)H * hs;                    // and its head-wrap carry
  // One chunk: its end, motion and (M-RoPE) section deltas through wave-uniform loads,
  // and this lane's pair frequency, all requested before the row loads, so the phases are
  // formed while the rows are in flight.
  const bool one = cm.num_chunks == 1;
  ChunkRef c1{0, 0, 0};
  int64_t sd[4] = {0, 0, 0, 0};
  if (one) {
    c1.end = cm.offsets[1];
    c1.delta = SEC ? chunk_moves(cm, 0) : cm.delta[0];
    if constexpr (SEC) {
#pragma unroll
      for (int k = 0; k < 4; ++k) sd[k] = k < cm.num_sections ? cm.delta[k] : 0;
    }
  }
  // More rows than one pass covers (only with more heads than a pass has rows): the
  // general loop, kept apart so that the common single pass below is straight-line code
  // (its row loads would otherwise wait on the frequency read at a loop header).
  const double om = lane < HALF ? ch.omega[lane] : 0.0;
  int p0 = 0;
  if (PAGED) {
    p0 = stage_block_table(cm, tb0, t1, sbt);
    __syncthreads();
  }
  // One pass over ROWS rows of the block (a lambda so that the common single-pass case
  // is straight-line code: a loop header makes the first row loads wait for earlier loads).
  auto pass = [&](int rbase, double om) {
    XV xv[UNR];
    uint32_t boff[UNR];  // byte offset of the lane's 8 elements, kOob = no row
    int tlk[UNR];  // token of each row group, relative to tb0
    const int R0 = rbase + wave * RPI + rr;
    int tl = R0 / H;
    int h = R0 - tl * H;
    uint32_t off = PAGED ? 0u : ((uint32_t)tb0 + (uint32_t)tl) * ss + (uint32_t)h * hs;
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      if (k > 0) {
        tl += dtl;
        h += dh;
        off += dstep;
        if (h >= H) {
          h -= H;
          ++tl;
          off += carry;
        }
      }
      bool ok = R0 + k * DR < nrows;
      tlk[k] = tl;
      uint32_t o = off;
      if constexpr (PAGED) {
        o = 0u;
        if (ok) {  // the staged table covers the block's own tokens only
          const int32_t so = slot32<true>(cm.page_size, cm.page_shift, sbt, p0, ps, (int32_t)ss,
                                          (int)tb0 + tl);
          ok = so >= 0;
          o = (uint32_t)so + (uint32_t)h * hs;
        }
      }
      boff[k] = ok ? (o + 8u * (uint32_t)q) * (uint32_t)sizeof(E) : kOob;
      bload_nt(rkv, boff[k], xv[k]);
    }
    // Token span of this wave's rows in this pass.
    const int r_first = rbase + wave * RPI;
    if (r_first >= nrows) return;
    const int r_last = min(nrows - 1, rbase + (wave + kWavesPerBlock * (UNR - 1)) * RPI + RPI - 1);
    int64_t t0 = tb0 + r_first / H;
    const int64_t tw1 = tb0 + r_last / H + 1;
    ChunkRef c = one ? c1 : find_chunk_wave<SEC ? 1 : 0>(cm, t0);
    while (true) {
      const int64_t s1 = min(tw1, c.end);
      if (s1 > t0 && c.delta != 0) {
        const int lo = (int)(t0 - tb0), hi = (int)(s1 - tb0);  // rows' tokens to store
        float2 own = make_float2(1.f, 0.f);
        if (lane < HALF) {
          int64_t d = c.delta;
          if constexpr (SEC) {
            if (one) {
              const int sec = section_of(cm, lane);
              d = sec == 0 ? sd[0] : sec == 1 ? sd[1] : sec == 2 ? sd[2] : sd[3];
            } else {
              d = pair_delta(cm, c, lane);
            }
          }
          own = phase_of(om, d);
        }
        float cs[8], sn[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int pi = IL ? fi0 + (e >> 1) : fi0 + e;
          cs[e] = __shfl(own.x, pi);
          sn[e] = (IL ? ((e & 1) ? 1.f : -1.f) : sgn) * __shfl(own.y, pi);
        }
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
          float a[8], b[8], y[8];
          unpack8(xv[k], a);
          if constexpr (IL) {
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = a[e ^ 1];
          } else {
            unpack8(lane_xor4<HX>(xv[k]), b);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = fmaf(a[e], cs[e], b[e] * sn[e]);
          XV o;
          if constexpr (Q) o = pack8_fp8(y);
          else o = pack8(y);
          if constexpr (SEC) o = keep_elems(o, xv[k], sn);
          bstore_nt(rkv, tlk[k] >= lo && tlk[k] < hi ? boff[k] : kOob, o);
        }
      }
      t0 = max(t0, s1);
      if (t0 >= tw1 || c.j + 1 >= cm.num_chunks) break;
      c = find_chunk_wave<SEC ? 1 : 0>(cm, t0, c.j + 1);
    }
  };
  if (nrows > ROWS) {
    for (int rbase = 0; rbase < nrows; rbase += ROWS) pass(rbase, ch.omega[lane < HALF ? lane : 0]);
    return;
  }
  pass(0, om);
}

// ------------------------------------------------------------------ rotation + patch (MFMA)

// Patch fragment of 8 consecutive k (bf16): a 16-byte load when all 8 lie below m and
// rows are 16-byte aligned (m % 8 == 0), else element loads with zero fill.
__device__ __forceinline__ u32x4_t load_frag(const uint16_t* row, int k0, int m, bool m8) {
  if (m8 && k0 + 8 <= m) return *(const u32x4_t*)(row + k0);
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (k0 + e < m) ? row[k0 + e] : (uint16_t)0;
  u32x4_t w;
  w.x = v[0] | ((uint32_t)v[1] << 16);
  w.y = v[2] | ((uint32_t)v[3] << 16);
  w.z = v[4] | ((uint32_t)v[5] << 16);
  w.w = v[6] | ((uint32_t)v[7] << 16);
  return w;
}

// Per-workgroup constants of the rotate+patch kernel that the tile loop reads.
template <bool Q>
struct PatchCtx {
  rsrc_t rkv;           // this layer of the channel (in place: read and written)
  rsrc_t rout;          // this layer of the destination (out of place)
  rsrc_t ru;            // U of this layer and channel
  uint32_t lane_b;      // byte offset of the lane's element (slot 0, head h, dim d0)
  uint32_t olane_b;     // same in the destination
  const uint16_t* Ul;   // U of this layer and channel
  const int* sbt;       // staged block table (paged)
  const int* osbt;      // staged destination block table (paged destination)
  int32_t page_stride, slot_stride;
  int32_t opage_stride, oslot_stride;
  int64_t tb0, t1;
  int p0, op0, m;
  int lane, wave, c16, g;
  int fi0;              // rotary pair of the lane's first dim (NeoX), or its first dim (IL)
  float sgn;
  bool lane_on, rot_lane;
  bool mixed;           // M-RoPE sections: some pairs may not turn
  float qs, qinv;       // fp8: the layer's dequantisation scale and its reciprocal
  int lend;             // pool order: end of the logical tokens the call covers
};

// KV, row offsets and U fragments of one 16-token tile of a wave.
template <bool Q, int MK>
struct Tile {
  typename Codec<Q>::XV x[4];
  // Byte offset of the lane's 8 elements of the row to store, kOob = none: in the
  // layer's source resource in place, in its destination resource out of place.
  uint32_t off[4];
  u32x4_t a[MK > 0 ? MK : 1];
};

// Token, inside a 16-token tile, of accumulator row 4g + i (lane group g = lane >> 4
// holds rows 4g .. 4g + 3 of its column): the A operand's row rho carries the U row of
// token tile_token(rho >> 2, rho & 3), so any one-to-one choice keeps the product right.
__device__ __forceinline__ int tile_token(int g, int i) { return g + 4 * i; }

// Loads tile kt (no rows when kt >= k_hi), keeping tokens in [t0, s1).  OUT: 0 in
// place, 1 contiguous destination, 2 paged destination; a row is loaded only when both
// its source and its destination slot exist.
template <bool Q, int MK, bool M8, bool PAGED, int OUT>
__device__ __forceinline__ void load_tile(const PatchCtx<Q>& c, const CommonArgs& cm, int kt,
                                          int k_hi, int64_t t0, int64_t s1, Tile<Q, MK>& T) {
  constexpr uint32_t es = sizeof(typename Codec<Q>::E);
  const int64_t ts = c.tb0 + 16 * (int64_t)kt;
  const bool tile_on = kt < k_hi;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = ts + tile_token(c.g, i);
    // Offsets only (no memory access depends on a branch): rows the lane skips load
    // zeros from and store nothing to offset kOob.
    uint32_t so = kOob, dso = kOob;
    if (tile_on && c.lane_on && t >= t0 && t < s1) {
      const int32_t s = slot32<PAGED>(cm.page_size, cm.page_shift, c.sbt, c.p0, c.page_stride,
                                      c.slot_stride, (int)t);
      if constexpr (OUT > 0) {
        const int32_t d = slot32<OUT == 2>(cm.out_page_size, cm.out_page_shift, c.osbt, c.op0,
                                           c.opage_stride, c.oslot_stride, (int)t);
        if (s >= 0 && d >= 0) {
          so = (uint32_t)s * es + c.lane_b;
          dso = (uint32_t)d * es + c.olane_b;
        }
      } else if (s >= 0) {
        so = (uint32_t)s * es + c.lane_b;
      }
    }
    T.off[i] = OUT > 0 ? dso : so;
    bload_nt(c.rkv, so, T.x[i]);
  }
  const int64_t tu = ts + tile_token(c.c16 >> 2, c.c16 & 3);
  const bool uok = tile_on && tu < c.t1;
#pragma unroll
  for (int ks = 0; ks < (MK > 0 ? MK : 1); ++ks) {
    T.a[ks] = u32x4_t{0u, 0u, 0u, 0u};
    if constexpr (MK > 0) {
      const int k0 = 32 * ks + 8 * c.g;
      if constexpr (M8) {
        // rows are 16-byte aligned; ranks past m read zeros
        const uint32_t uo = uok && k0 < c.m ? ((uint32_t)tu * c.m + k0) * 2u : kOob;
        T.a[ks] = bload(c.ru, uo);
      } else if (uok) {
        T.a[ks] = load_frag(c.Ul + tu * c.m, k0, c.m, false);
      }
    }
  }
  // The tile's requests leave together: the scheduler would otherwise sink the later U
  // loads below the first waits on row data, serialising their latency.
  __builtin_amdgcn_sched_barrier(0);
}

// Pool order (in place, one chunk, pages of a multiple of 16 slots): the workgroup's
// "tokens" are pool slots, so a tile is 16 consecutive slots of one page.  sbt holds
// the logical page of each of the workgroup's pool pages (-1: the page holds none of
// the call's tokens).  Row addresses come straight from the slot; only validity and the
// U rows depend on the logical page.
// KV rows of tile kt, loaded by pool slot alone, before the logical pages are known:
// every row of the tile is requested (past the tile range: none) and stored nowhere until
// pool_validate has seen its page.
template <bool Q, int MK>
__device__ __forceinline__ void pool_rows(const PatchCtx<Q>& c, const CommonArgs& cm, int kt,
                                          int k_hi, Tile<Q, MK>& T) {
  constexpr uint32_t es = sizeof(typename Codec<Q>::E);
  const int ps = (int)c.tb0 + 16 * kt;  // pool slot of the tile's first row
  const int P = cm.page_size;
  const int pg = cm.page_shift >= 0 ? ps >> cm.page_shift : ps / P;
  const int si = ps - pg * P;
  const uint32_t rowb = (uint32_t)pg * (uint32_t)c.page_stride + (uint32_t)si * c.slot_stride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t so = kt < k_hi && c.lane_on
                            ? (rowb + (uint32_t)tile_token(c.g, i) * c.slot_stride) * es + c.lane_b
                            : kOob;
    T.off[i] = kOob;
    bload_nt(c.rkv, so, T.x[i]);
  }
}

// Logical page of the pool page that holds tile kt (-1: none of the call's tokens), read
// with a wave-uniform load; in the prologue, before any store, that is a scalar load, which
// waits on its own counter rather than behind the wave's row loads.
template <bool Q>
__device__ __forceinline__ int pool_lpage(const PatchCtx<Q>& c, const CommonArgs& cm, int kt,
                                          int k_hi) {
  if (kt >= k_hi) return -1;
  const int ps = (int)c.tb0 + 16 * kt;
  const int pg = cm.page_shift >= 0 ? ps >> cm.page_shift : ps / cm.page_size;
  const int32_t* __restrict__ inv = cm.inv;
  const int v = inv[__builtin_amdgcn_readfirstlane(pg)];
  return v >= 0 && v < cm.num_logical_pages ? v : -1;
}

// Store offsets and U rows of tile kt, whose pool page holds logical page lp: rows of a
// page that holds none of the call's tokens, or tokens at or past lend, are not stored.
// With LOAD the KV rows are requested here as well, only for those rows.
template <bool Q, int MK, bool M8, bool LOAD>
__device__ __forceinline__ void pool_validate(const PatchCtx<Q>& c, const CommonArgs& cm, int kt,
                                              int lp, Tile<Q, MK>& T) {
  constexpr uint32_t es = sizeof(typename Codec<Q>::E);
  const int ps = (int)c.tb0 + 16 * kt;
  const int P = cm.page_size;
  const int pg = cm.page_shift >= 0 ? ps >> cm.page_shift : ps / P;
  const int si = ps - pg * P;
  // Logical token of the first row (tuned kernels keep token ids below 2^30); a page no
  // entry names gives lend, so that none of its rows is stored.
  const int tl = lp >= 0 ? lp * P + si : c.lend;
  const uint32_t rowb = (uint32_t)pg * (uint32_t)c.page_stride + (uint32_t)si * c.slot_stride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = tile_token(c.g, i);
    uint32_t so = kOob;
    if (c.lane_on && tl + r < c.lend) so = (rowb + (uint32_t)r * c.slot_stride) * es + c.lane_b;
    T.off[i] = so;
    if constexpr (LOAD) bload_nt(c.rkv, so, T.x[i]);
  }
  const int tu = tl + tile_token(c.c16 >> 2, c.c16 & 3);
  const bool uok = tu < (int)cm.total_tokens;
#pragma unroll
  for (int ks = 0; ks < (MK > 0 ? MK : 1); ++ks) {
    T.a[ks] = u32x4_t{0u, 0u, 0u, 0u};
    if constexpr (MK > 0) {
      const int k0 = 32 * ks + 8 * c.g;
      if constexpr (M8) {
        const uint32_t uo = uok && k0 < c.m ? ((uint32_t)tu * c.m + k0) * 2u : kOob;
        T.a[ks] = bload(c.ru, uo);
      } else if (uok) {
        T.a[ks] = load_frag(c.Ul + tu * c.m, k0, c.m, false);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // the tile's requests leave together
}

// Rotates, patches and stores a loaded tile.  HX is the NeoX partner lane distance, -1
// for interleaved pairs (partner in the other half of the same word), 0 for no
// rotation.  Lane l holds features fb + 8c + n (c = l & 15, n < 8) of tokens
// 4g .. 4g + 3 (g = l >> 4).
//
// Patch on MFMA 16x16x32 bf16: D[t][col] = C[t][col] + sum_k A[t][k] B[k][col] with
// A = U rows (tokens), B = V^T.  Column col of MFMA tile n is feature fb + 8 col + n,
// so the output layout (lane l holds rows 4g..4g+3 of column l & 15) is the lane's own
// feature n of its 4 tokens: the rotated values are the C operand and the result is
// already where it is stored.  Output tiles go two at a time (features 2p, 2p + 1 form
// one packed bf16 pair), so only 8 accumulators are live.
//
// Phases sit in LDS as (cos, sin) per rotary pair.  With M-RoPE sections a pair whose
// section delta is 0 has sin exactly 0 and is not rotated.
//
// fp8 (Q): the rotation runs on code values and the result is rotated + patch * (1/s)
// with the patch in value units.  At MK = 1 the MFMA starts from a zero accumulator and
// one FMA finishes each element; at larger MK, where the rotated values cannot stay
// live beside the accumulators without spilling, the accumulator starts at s * rotated
// and the sum is multiplied by 1/s.
// Rotated (or unrotated) values r0, r1 of features 2pp, 2pp + 1 of the lane's 4 tokens,
// and whether each of the two features turns.  Phases sit in LDS as (cos, sin) per
// rotary pair; with M-RoPE sections a pair whose section delta is 0 has sin exactly 0
// and is not rotated.
template <bool Q, int HX>
__device__ __forceinline__ void rotate_pair(const PatchCtx<Q>& c, const float4* sph2,
                                            const typename Codec<Q>::XV (&x)[4], int pp,
                                            float (&r0)[4], float (&r1)[4], bool& turn0,
                                            bool& turn1) {
  using P = Codec<Q>;
  const float2* sph = reinterpret_cast<const float2*>(sph2);
  float4 ph = make_float4(1.f, 0.f, 1.f, 0.f);
  if constexpr (HX > 0) ph = sph2[(c.fi0 >> 1) + pp];
  if constexpr (HX < 0) {
    const float2 q = sph[(c.fi0 >> 1) + pp];
    ph = make_float4(q.x, q.y, q.x, q.y);
  }
  turn0 = HX != 0 && c.rot_lane && !(c.mixed && ph.y == 0.f);
  turn1 = HX != 0 && c.rot_lane && !(c.mixed && ph.w == 0.f);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = P::word(x[i], pp);
    const float2 av = P::pair(w, pp);
    const float a0 = av.x, a1 = av.y;
    float y0 = a0, y1 = a1;
    if constexpr (HX > 0) {
      const float2 bv = P::pair(lane_xor<HX>(w), pp);
      y0 = fmaf(a0, ph.x, bv.x * (c.sgn * ph.y));
      y1 = fmaf(a1, ph.z, bv.y * (c.sgn * ph.w));
    } else if constexpr (HX < 0) {
      y0 = fmaf(a0, ph.x, -(a1 * ph.y));
      y1 = fmaf(a1, ph.x, a0 * ph.y);
    }
    r0[i] = turn0 ? y0 : a0;
    r1[i] = turn1 ? y1 : a1;
  }
}

template <bool Q, int MK, int HX, int OUT>
__device__ __forceinline__ void finish_tile(const PatchCtx<Q>& c, const u32x4_t* sV,
                                            const float4* sph2, Tile<Q, MK>& T) {
  using P = Codec<Q>;
  {
    // bf16: feature pair pp of a row is one word, read (with the partner lane's word)
    // before its result is written, so results overwrite the loaded words.  fp8 packs
    // two pairs per word and keeps a separate result.
    typename P::XV outq[4];
    typename P::XV* out = Q ? outq : T.x;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {  // features 2pp, 2pp + 1 of the lane's 8
      float r0[4], r1[4];
      bool turn0, turn1;
      rotate_pair<Q, HX>(c, sph2, T.x, pp, r0, r1, turn0, turn1);
      if constexpr (MK == 0) {
        // No patch (out of place only): rotated dims are rounded once, every other
        // element is copied bit for bit.
#pragma unroll
        for (int i = 0; i < 4; ++i)
          P::put_keep(out[i], T.x[i], pp, r0[i], r1[i], !turn0, !turn1);
      } else {
        constexpr bool kFmaScale = Q && MK == 1;
        f32x4_t acc0, acc1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc0[i] = kFmaScale ? 0.f : Q ? r0[i] * c.qs : r0[i];
          acc1[i] = kFmaScale ? 0.f : Q ? r1[i] * c.qs : r1[i];
        }
#pragma unroll
        for (int ks = 0; ks < MK; ++ks) {
          const bf16x8_t A = __builtin_bit_cast(bf16x8_t, T.a[ks]);
          const bf16x8_t B0 = __builtin_bit_cast(bf16x8_t, sV[((2 * pp) * MK + ks) * 64 + c.lane]);
          const bf16x8_t B1 =
              __builtin_bit_cast(bf16x8_t, sV[((2 * pp + 1) * MK + ks) * 64 + c.lane]);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B0, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B1, acc1, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          P::put(out[i], pp,
                 kFmaScale ? fmaf(acc0[i], c.qinv, r0[i]) : Q ? acc0[i] * c.qinv : acc0[i],
                 kFmaScale ? fmaf(acc1[i], c.qinv, r1[i]) : Q ? acc1[i] * c.qinv : acc1[i]);
      }
      // Keep the scheduler from hoisting every feature pair's LDS reads at once (it
      // would hold all B fragments live and lower the occupancy).
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) bstore_nt(OUT > 0 ? c.rout : c.rkv, T.off[i], out[i]);
  }
}

// The same tile with the patch on VALU instead of MFMA (bf16 in place; a measurement
// variant for the MFMA-versus-VALU comparison): the rank-m sum of the lane's 4 tokens x
// 8 features is taken with v_dot2_f32_bf16 (two bf16 products per instruction, fp32
// accumulation) from the tile's U rows, written per wave to LDS from the A fragments
// (lane (c16, g) holds U[c16][32 ks + 8 g ...]), and the staged V rows (the B fragment
// of feature n, rank step ks, lane group g holds V[n][32 ks + 8 g ...]).
template <int MK, int HX>
__device__ __forceinline__ void finish_tile_valu(const PatchCtx<false>& c, const u32x4_t* sV,
                                                 const float4* sph2, u32x4_t* sUw,
                                                 Tile<false, MK>& T) {
  using P = Codec<false>;
  constexpr int UR = 4 * MK + 1;  // 16-byte words per staged U row (+1 spreads banks)
#pragma unroll
  for (int ks = 0; ks < MK; ++ks) sUw[c.c16 * UR + 4 * ks + c.g] = T.a[ks];
  float acc[4][8];  // token 4g + i, feature 8c16 + e
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    float r0[4], r1[4];
    bool turn0, turn1;
    rotate_pair<false, HX>(c, sph2, T.x, pp, r0, r1, turn0, turn1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i][2 * pp] = r0[i];
      acc[i][2 * pp + 1] = r1[i];
    }
  }
#pragma unroll
  for (int q = 0; q < 4 * MK; ++q) {  // rank steps of 8
    if (8 * q >= c.m) break;
    u32x4_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = sUw[(4 * c.g + i) * UR + q];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const u32x4_t v = sV[(e * MK + (q >> 2)) * 64 + (q & 3) * 16 + c.c16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // Words go through scalars: a bit cast taken directly of a vector element
          // (u[i][w]) reads element 0 for every w with this compiler.
          const uint32_t uw = u[i][w], vw = v[w];
          acc[i][e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, uw),
                                                      __builtin_bit_cast(bf16x2_t, vw),
                                                      acc[i][e], false);
        }
    }
  }
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int i = 0; i < 4; ++i) P::put(T.x[i], pp, acc[i][2 * pp], acc[i][2 * pp + 1]);
#pragma unroll
  for (int i = 0; i < 4; ++i) bstore_nt(c.rkv, T.off[i], T.x[i]);
}

// The wave's 16-token tiles (kt = wave mod 4, kt + 4, ...) that meet [t0, s1), one at a
// time; only tokens in [t0, s1) are loaded and stored.  When `use_pre`, A already holds
// the wave's first tile (loaded before the workgroup staged the chunk).
// VALU: the patch on VALU (finish_tile_valu, with the wave's U staging area sUw).
template <bool Q, int MK, bool M8, bool PAGED, int HX, int OUT, bool VALU>
__device__ __forceinline__ void patch_tiles(const PatchCtx<Q>& c, const CommonArgs& cm,
                                            const u32x4_t* sV, const float4* sph2,
                                            u32x4_t* sUw, int64_t t0, int64_t s1,
                                            Tile<Q, MK>& A, bool use_pre) {
  constexpr int W = kWavesPerBlock;
  const int k_lo = (int)((t0 - c.tb0) >> 4);
  const int k_hi = (int)((s1 - c.tb0 + 15) >> 4);
  int kt = k_lo + ((c.wave - k_lo) % W + W) % W;
  auto finish = [&]() {
    if constexpr (VALU) finish_tile_valu<MK, HX>(c, sV, sph2, sUw, A);
    else finish_tile<Q, MK, HX, OUT>(c, sV, sph2, A);
  };
  if (use_pre) {
    finish();
    kt += W;
  }
  for (; kt < k_hi; kt += W) {
    load_tile<Q, MK, M8, PAGED, OUT>(c, cm, kt, k_hi, t0, s1, A);
    finish();
  }
}

// One chunk, logical order: the wave's tiles kt = wave, wave + 4, ... up to the chunk's
// end s1; A holds the first NT of them already (in flight together), the rest follow one
// at a time.
template <bool Q, int MK, bool M8, bool PAGED, int HX, int OUT, int NT>
__device__ __forceinline__ void patch_tiles_batch(const PatchCtx<Q>& c, const CommonArgs& cm,
                                                  const u32x4_t* sV, const float4* sph2,
                                                  int64_t s1, Tile<Q, MK> (&A)[NT]) {
  const int k_hi = (int)((s1 - c.tb0 + 15) >> 4);
#pragma unroll
  for (int i = 0; i < NT; ++i) finish_tile<Q, MK, HX, OUT>(c, sV, sph2, A[i]);
  for (int kt = c.wave + kWavesPerBlock * NT; kt < k_hi; kt += kWavesPerBlock) {
    load_tile<Q, MK, M8, PAGED, OUT>(c, cm, kt, k_hi, c.tb0, s1, A[0]);
    finish_tile<Q, MK, HX, OUT>(c, sV, sph2, A[0]);
  }
}

// Pool order: the wave's tiles kt = wave, wave + 4, ... of the workgroup's slot range;
// A holds the first NT of them already (in flight together), the rest follow one at a
// time.
template <bool Q, int MK, bool M8, int HX, int NT>
__device__ __forceinline__ void patch_tiles_pool(const PatchCtx<Q>& c, const CommonArgs& cm,
                                                 const u32x4_t* sV, const float4* sph2,
                                                 int k_hi, Tile<Q, MK> (&A)[NT]) {
#pragma unroll
  for (int i = 0; i < NT; ++i) finish_tile<Q, MK, HX, 0>(c, sV, sph2, A[i]);
  for (int kt = c.wave + kWavesPerBlock * NT; kt < k_hi; kt += kWavesPerBlock) {
    pool_validate<Q, MK, M8, true>(c, cm, kt, pool_lpage(c, cm, kt, k_hi), A[0]);
    finish_tile<Q, MK, HX, 0>(c, sV, sph2, A[0]);
  }
}

// Workgroup = one 128-feature block of one channel and layer over `block_tokens` tokens;
// wave w takes the 16-token tiles w, w + 4, ....  The chunk the workgroup works on is
// staged once in LDS (the B fragments of its feature factor, the phases of its delta),
// then the waves stream their tiles of that chunk.  Workgroups are numbered so that all
// feature blocks of one token group run on the same XCD (consecutive workgroup ids go
// to consecutive XCDs), where they share the token group's U rows in that XCD's L2.
//
// TAIL = false covers every token group from its first token to the end of the chunk
// that holds it (all of it in the common case of a group inside one chunk); in place,
// when the grid holds units past the token groups, unit k - 1 covers chunk k's part of
// the group that chunk k's first token cuts, so one launch covers the call.  TAIL =
// true covers the rest of the groups that a chunk boundary cuts otherwise: the grid
// runs over boundaries (cm.tail_mode == 1: unit k handles boundary offsets[k + 1] when
// it is the first boundary inside its group) or over groups (cm.tail_mode == 2, when
// chunks outnumber groups).  Keeping that loop over chunks in its own kernel keeps the
// common kernel's register count (and so its occupancy) down.
//
// OUT != 0 is the out-of-place form (recall): rows are read through the source layout
// and whole result rows written through the destination layout (OUT 1 contiguous, 2
// paged); MK = 0 is its no-patch form.  Q: fp8 E4M3 elements (bf16 factors).  VALU
// (bf16 in place, head launch): the patch on VALU instead of MFMA, for measurement.
template <bool Q, int MK, bool M8, bool PAGED, bool TAIL, int OUT, bool VALU = false,
          bool POOL = false, int NT = 1, int CH = 0>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(TAIL || MK > 2 || (MK == 2 && OUT != 0) ? 1 : NT > 1 ? 3 : 4)))
void relocate_patch_rows(ChanArgs ch0, ChanArgs ch1, CommonArgs cm, int64_t blocks_per_layer,
                         int xcd_group) {
  __shared__ u32x4_t sV[8 * (MK > 0 ? MK : 1) * 64];
  __shared__ float4 sph2[kMaxTunedHalf / 2];  // (cos, sin) of pairs 2p and 2p + 1
  __shared__ int sbt[kMaxBlockTokens + 1];
  __shared__ int osbt[OUT == 2 ? kMaxBlockTokens + 1 : 1];
  __shared__ u32x4_t sUv[VALU ? kWavesPerBlock * 16 * (4 * MK + 1) : 1];
  const int lane = threadIdx.x & 63;
  u32x4_t* sUw = sUv + (VALU ? (threadIdx.x >> 6) * 16 * (4 * MK + 1) : 0);

  // Logical workgroup index: groups of 8 * xcd_group ids are permuted so that XCD x
  // gets xcd_group consecutive logical blocks (one token group's feature blocks).
  int64_t bid = blockIdx.x;
  if (xcd_group > 0) {
    const int64_t G = 8 * (int64_t)xcd_group;
    const int64_t full = ((int64_t)gridDim.x / G) * G;
    if (bid < full) {
      const int64_t i = bid % G;
      bid = bid - i + (i % 8) * xcd_group + i / 8;
    }
  }
  // grid < 2^32 workgroups: 32-bit division
  const uint32_t bpl = (uint32_t)blocks_per_layer;
  const int64_t layer = (uint32_t)bid / bpl;
  int64_t b = (uint32_t)bid - (uint32_t)layer * bpl;
  const bool second = b >= ch0.blocks;
  if (second) b -= ch0.blocks;
  // Field-wise choice of the channel (a reference to either argument would copy both
  // to scratch memory).
#define KAMERA_CH(f) (second ? ch1.f : ch0.f)
  const int fblocks = KAMERA_CH(fblocks);
  const int64_t tg = (uint32_t)b / (uint32_t)fblocks;
  const int fbk = (int)(b - tg * fblocks);

  using E = typename Codec<Q>::E;
  PatchCtx<Q> c;
  c.lane = lane;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar tile indices
  c.c16 = lane & 15;
  c.g = lane >> 4;
  c.m = cm.rank;
  const int m = cm.rank;
  const int D = KAMERA_CH(dim);
  const int r = KAMERA_CH(rope_dim);
  const int F = KAMERA_CH(heads) * D;
  const int fb = fbk * 128;
  const int f0 = fb + 8 * c.c16;
  c.lane_on = f0 < F;
  const int h = f0 / D;
  const int d0 = f0 - h * D;
  c.rot_lane = c.lane_on && d0 < r;
  const bool il = cm.pairing == 1;
  c.fi0 = il ? d0 : (d0 < (r >> 1) ? d0 : d0 - (r >> 1));
  c.sgn = d0 < (r >> 1) ? -1.f : 1.f;
  c.mixed = cm.num_sections > 1;
  const int hx = il ? -1 : r >> 4;  // NeoX partner lane distance half / 8; -1 interleaved

  c.slot_stride = (int32_t)KAMERA_CH(slot_stride);
  c.page_stride = (int32_t)KAMERA_CH(page_stride);
  c.rkv = make_rsrc((E*)KAMERA_CH(data) + layer * KAMERA_CH(layer_stride),
                    KAMERA_CH(layer_bytes));
  c.lane_b = (uint32_t)(((int64_t)h * KAMERA_CH(head_stride) + d0) * (int64_t)sizeof(E));
  c.qs = c.qinv = 1.f;
  if constexpr (Q) {
    c.qs = KAMERA_CH(scale)[layer];
    c.qinv = 1.f / c.qs;
  }
  c.rout = c.rkv;
  c.olane_b = 0;
  c.opage_stride = c.oslot_stride = 0;
  if constexpr (OUT > 0) {
    c.rout = make_rsrc((E*)KAMERA_CH(out) + layer * KAMERA_CH(out_layer_stride),
                       KAMERA_CH(out_layer_bytes));
    c.olane_b =
        (uint32_t)(((int64_t)h * KAMERA_CH(out_head_stride) + d0) * (int64_t)sizeof(E));
    c.oslot_stride = (int32_t)KAMERA_CH(out_slot_stride);
    c.opage_stride = (int32_t)KAMERA_CH(out_page_stride);
  }
  c.Ul = (const uint16_t*)KAMERA_CH(U) + layer * cm.total_tokens * m;
  c.ru = make_rsrc(c.Ul, KAMERA_CH(u_layer_bytes));
  const uint16_t* Vl = (const uint16_t*)KAMERA_CH(V) + layer * (int64_t)cm.num_chunks * F * m;

  // Token group and the first token this workgroup works on.
  [[maybe_unused]] int64_t start;
  [[maybe_unused]] int from = 0;  // chunk index to search from
  if constexpr (TAIL) {
    if (cm.tail_mode == 1) {
      const int k = (int)tg + 1;  // boundary offsets[k], 1 <= k < num_chunks
      const int64_t o = cm.offsets[k];
      const int64_t g = o / cm.block_tokens;
      c.tb0 = g * cm.block_tokens;
      c.t1 = min(c.tb0 + (int64_t)cm.block_tokens, cm.total_tokens);
      // Only the first boundary strictly inside the group starts work there.
      if (!(o > c.tb0 && o < c.t1) || cm.offsets[k - 1] > c.tb0) return;
      start = o;
      from = k;
    } else {
      c.tb0 = tg * cm.block_tokens;
      c.t1 = min(c.tb0 + (int64_t)cm.block_tokens, cm.total_tokens);
      const ChunkRef first = find_chunk_wave(cm, c.tb0);
      if (first.end <= c.tb0 || first.end >= c.t1) return;  // no boundary inside
      start = first.end;
      from = first.j + 1;
    }
  } else if (!POOL && CH != 1 && OUT == 0 && tg >= cm.token_groups) {
    // A boundary unit of a head launch over several chunks: unit k - 1 covers chunk k's
    // part of the token group that its first token offsets[k] cuts, [offsets[k],
    // min(offsets[k + 1], group end)).  Boundaries on a group's first token and empty
    // chunks leave it idle; the group's head unit covers its part up to its first chunk
    // end, so the units of a group cover it once.
    const int k = (int)(tg - cm.token_groups) + 1;  // 1 <= k < num_chunks
    const int64_t o = cm.offsets[k];
    const int64_t g0 = o / cm.block_tokens * cm.block_tokens;
    c.tb0 = o;
    c.t1 = min(g0 + (int64_t)cm.block_tokens, cm.total_tokens);
    if (o <= g0 || o >= c.t1 || cm.offsets[k + 1] <= o) return;
    start = o;
  } else {
    // Pool order: the workgroup covers pool slots [tb0, t1) of num_pages * page_size.
    c.tb0 = tg * cm.block_tokens;
    c.t1 = min(c.tb0 + (int64_t)cm.block_tokens, POOL ? cm.pool_slots : cm.total_tokens);
    start = c.tb0;
  }
  c.p0 = 0;
  c.op0 = 0;
  c.sbt = sbt;
  c.osbt = osbt;
  c.lend = (int)cm.total_tokens;

  // B fragments of chunk j's feature factor into sV: thread item u of 2 * MK is sV[u *
  // kBlock + threadIdx.x], feature fb + 8 (lane & 15) + n, ranks 32 ks + 8 (lane >> 4) ..
  // + 7 with n * MK + ks = 4 u + wave.  Rows 16-byte aligned (M8): each item is one
  // 16-byte load straight into LDS (past the factor's range it reads zeros), no
  // registers held; the workgroup barrier's release waits for them.  Otherwise through
  // registers.
  auto stage_factor = [&](int j) {
    const uint16_t* Vj = Vl + (int64_t)j * F * m;
    if constexpr (M8 && MK > 0) {
      const rsrc_t rv = make_rsrc(Vj, (uint32_t)((int64_t)F * m * 2));
#pragma unroll
      for (int u = 0; u < 2 * MK; ++u) {
        const int nk = 4 * u + c.wave;  // n * MK + ks
        const int n = nk / MK;
        const int ks = nk - n * MK;
        const int f = fb + 8 * c.c16 + n;
        const int k0 = 32 * ks + 8 * c.g;
        const uint32_t off = f < F && k0 < m ? ((uint32_t)f * (uint32_t)m + (uint32_t)k0) * 2u : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (__attribute__((address_space(3))) void*)(sV + kBlock * u + 64 * c.wave), 16, off,
            0, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 2 * MK; ++u) {  // none when MK == 0
        const int it = threadIdx.x + kBlock * u;
        const int l = it & 63;
        const int nk = it >> 6;  // n * MK + ks
        const int n = nk / (MK > 0 ? MK : 1);
        const int ks = nk - n * MK;
        const int f = fb + 8 * (l & 15) + n;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (f < F) v = load_frag(Vj + (int64_t)f * m, 32 * ks + 8 * (l >> 4), m, M8);
        sV[it] = v;
      }
    }
  };
  // One pair frequency per thread; (cos, sin) of pairs 2p and 2p + 1 are adjacent.
  auto phases = [&](const ChunkRef& ck) {
    if (threadIdx.x < (r >> 1))
      reinterpret_cast<float2*>(sph2)[threadIdx.x] =
          phase_of(KAMERA_CH(omega[threadIdx.x]), pair_delta(cm, ck, threadIdx.x));
  };
  // Stages chunk j's B fragments (and, when rotating, its phases) in LDS.
  auto stage = [&](const ChunkRef& ck, bool rotate) {
    stage_factor(ck.j);
    if (rotate) phases(ck);
  };
#define KAMERA_PATCH_SWITCH(USE)                                                                   \
  switch (rotate ? hx : 0) {                                                                       \
    case 1: patch_tiles<Q, MK, M8, PAGED, 1, OUT, VALU>(c, cm, sV, sph2, sUw, t0, s1, A, USE); break;   \
    case 2: patch_tiles<Q, MK, M8, PAGED, 2, OUT, VALU>(c, cm, sV, sph2, sUw, t0, s1, A, USE); break;   \
    case 4: patch_tiles<Q, MK, M8, PAGED, 4, OUT, VALU>(c, cm, sV, sph2, sUw, t0, s1, A, USE); break;   \
    case 8: patch_tiles<Q, MK, M8, PAGED, 8, OUT, VALU>(c, cm, sV, sph2, sUw, t0, s1, A, USE); break;   \
    case -1: patch_tiles<Q, MK, M8, PAGED, -1, OUT, VALU>(c, cm, sV, sph2, sUw, t0, s1, A, USE); break; \
    default: patch_tiles<Q, MK, M8, PAGED, 0, OUT, VALU>(c, cm, sV, sph2, sUw, t0, s1, A, USE); break;  \
  }

  // A head launch over one chunk needs no chunk lookup: the chunk's feature factor is
  // requested before anything else (straight into LDS), so the workgroup's wait for it
  // overlaps the table staging and the first tiles' loads instead of queueing behind them.
  // CH: 1 the launch moves one chunk, 2 several, 0 decided here (the batched head
  // launches are compiled for one case each, so neither path's registers burden the other).
  const bool one = CH == 1 ? true : CH == 2 ? false : !TAIL && cm.num_chunks == 1;
  // Wave-uniform lookups first, while nothing has been written yet (the compiler then
  // makes them scalar loads, which do not wait behind the row loads): chunk 0's end and
  // motion, and in pool order the logical page of each of the wave's first NT tiles.
  ChunkRef ck0{0, 0, 0};
  int64_t sd[4] = {0, 0, 0, 0};  // M-RoPE: chunk 0's section deltas
  if (one) {
    ck0.end = cm.offsets[1];
    ck0.delta = chunk_moves(cm, 0);
    if (cm.num_sections > 1) {
#pragma unroll
      for (int k = 0; k < 4; ++k) sd[k] = k < cm.num_sections ? cm.delta[k] : 0;
    }
    if (POOL) c.lend = (int)max(min(ck0.end, cm.total_tokens), (int64_t)0);
  }
  // This thread's pair frequency (a per-thread read of the argument block: issued before
  // the row loads, so waiting for it does not wait for them).
  double om = 0.0;
  if (!TAIL && threadIdx.x < (r >> 1)) {
    if (second) om = ch1.omega[threadIdx.x];
    else om = ch0.omega[threadIdx.x];
  }
  int lps[NT];
  if (POOL) {
    const int k_hi = (int)((c.t1 - c.tb0 + 15) >> 4);
#pragma unroll
    for (int i = 0; i < NT; ++i) lps[i] = pool_lpage(c, cm, c.wave + kWavesPerBlock * i, k_hi);
  }
  if (one && M8) stage_factor(0);
  // Pool order: the first tile's rows are requested by pool slot right away, before the
  // logical pages (needed only for validity and the U rows) arrive.
  // The wave's first NT tiles, requested together (one chunk); A is the first.
  Tile<Q, MK> TB[NT];
  Tile<Q, MK>& A = TB[0];
  if (POOL) {
    const int k_hi = (int)((c.t1 - c.tb0 + 15) >> 4);
#pragma unroll
    for (int i = 0; i < NT; ++i) pool_rows<Q, MK>(c, cm, c.wave + kWavesPerBlock * i, k_hi, TB[i]);
  } else if (PAGED) {
    c.p0 = stage_block_table(cm, c.tb0, c.t1, sbt);
  }
  if (OUT == 2)
    c.op0 = stage_table(cm.out_block_table, cm.out_num_pages, cm.out_page_size, c.tb0, c.t1, osbt);
  if ((PAGED && !POOL) || OUT == 2) __syncthreads();  // staged tables

  if constexpr (!TAIL) {
    const int ntiles = (int)((c.t1 - c.tb0 + 15) >> 4);
    if (one) {
      if constexpr (POOL) {
        // Rows of pool pages that hold none of the call's tokens are left alone.
#pragma unroll
        for (int i = 0; i < NT; ++i)
          pool_validate<Q, MK, M8, false>(c, cm, c.wave + kWavesPerBlock * i, lps[i], TB[i]);
      } else {
#pragma unroll
        for (int i = 0; i < NT; ++i)
          load_tile<Q, MK, M8, PAGED, OUT>(c, cm, c.wave + kWavesPerBlock * i, ntiles, c.tb0,
                                           c.t1, TB[i]);
      }
      const ChunkRef ck = ck0;
      if constexpr (!POOL) {
        if (min(c.t1, ck.end) <= c.tb0) return;  // offsets that do not cover the group
#pragma unroll
        for (int b = 0; b < NT; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (c.tb0 + 16 * (c.wave + kWavesPerBlock * b) + tile_token(c.g, i) >= ck.end)
              TB[b].off[i] = kOob;
      }
      const bool rotate = r > 0 && ck.delta != 0;
      if (!M8) stage_factor(0);
      if (rotate && threadIdx.x < (r >> 1)) {
        // chunk 0's phases from the uniform loads above
        int64_t d = ck.delta;
        if (cm.num_sections > 1) {
          const int sec = section_of(cm, threadIdx.x);
          d = sec == 0 ? sd[0] : sec == 1 ? sd[1] : sec == 2 ? sd[2] : sd[3];
        }
        reinterpret_cast<float2*>(sph2)[threadIdx.x] = phase_of(om, d);
      }
      __syncthreads();
      if constexpr (POOL) {
        switch (rotate ? hx : 0) {
          case 1: patch_tiles_pool<Q, MK, M8, 1, NT>(c, cm, sV, sph2, ntiles, TB); break;
          case 2: patch_tiles_pool<Q, MK, M8, 2, NT>(c, cm, sV, sph2, ntiles, TB); break;
          case 4: patch_tiles_pool<Q, MK, M8, 4, NT>(c, cm, sV, sph2, ntiles, TB); break;
          case 8: patch_tiles_pool<Q, MK, M8, 8, NT>(c, cm, sV, sph2, ntiles, TB); break;
          case -1: patch_tiles_pool<Q, MK, M8, -1, NT>(c, cm, sV, sph2, ntiles, TB); break;
          default: patch_tiles_pool<Q, MK, M8, 0, NT>(c, cm, sV, sph2, ntiles, TB); break;
        }
      } else if constexpr (NT > 1) {
        const int64_t s1 = min(c.t1, ck.end);
        switch (rotate ? hx : 0) {
          case 1: patch_tiles_batch<Q, MK, M8, PAGED, 1, OUT, NT>(c, cm, sV, sph2, s1, TB); break;
          case 2: patch_tiles_batch<Q, MK, M8, PAGED, 2, OUT, NT>(c, cm, sV, sph2, s1, TB); break;
          case 4: patch_tiles_batch<Q, MK, M8, PAGED, 4, OUT, NT>(c, cm, sV, sph2, s1, TB); break;
          case 8: patch_tiles_batch<Q, MK, M8, PAGED, 8, OUT, NT>(c, cm, sV, sph2, s1, TB); break;
          case -1: patch_tiles_batch<Q, MK, M8, PAGED, -1, OUT, NT>(c, cm, sV, sph2, s1, TB); break;
          default: patch_tiles_batch<Q, MK, M8, PAGED, 0, OUT, NT>(c, cm, sV, sph2, s1, TB); break;
        }
      } else {
        const int64_t t0 = c.tb0, s1 = min(c.t1, ck.end);
        KAMERA_PATCH_SWITCH(true)
      }
    } else if constexpr (!POOL) {
      // Several chunks.  The chunk lookup's loads go out first (lane k reads chunk k's end
      // and motion), then the wave's first NT tiles up to the group's end, so resolving
      // the chunk waits for the lookup alone; rows past the chunk's end are then dropped
      // (the tail launch covers them).
      const int n = cm.num_chunks;
      int64_t e0 = INT64_MAX, d0 = 0;
      if (lane < n) {
        e0 = cm.offsets[lane + 1];
        d0 = chunk_moves(cm, lane);
      }
#pragma unroll
      for (int b = 0; b < NT; ++b)
        load_tile<Q, MK, M8, PAGED, OUT>(c, cm, c.wave + kWavesPerBlock * b, ntiles, c.tb0, c.t1,
                                         TB[b]);
      ChunkRef ck{0, 0, 0};
      const int cnt = __popcll(__ballot(e0 <= c.tb0));  // chunks that end at or before tb0
      if (cnt < 64 || n <= 64) {
        const int src = cnt < 64 ? cnt : 63;
        ck.j = min(src, n - 1);
        ck.end = __shfl(e0, src);
        ck.delta = __shfl(d0, src);
        if (src >= n) {  // past the last chunk: clamp to it
          ck.j = n - 1;
          ck.end = cm.offsets[n];
          ck.delta = chunk_moves(cm, n - 1);
        }
      } else {
        ck = find_chunk_wave(cm, c.tb0, 64);
      }
      const int64_t t0 = c.tb0, s1 = min(c.t1, ck.end);
      if (s1 <= t0) return;  // offsets that do not cover the group: nothing here
#pragma unroll
      for (int b = 0; b < NT; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c.tb0 + 16 * (c.wave + kWavesPerBlock * b) + tile_token(c.g, i) >= s1)
            TB[b].off[i] = kOob;
      const bool rotate = r > 0 && ck.delta != 0;
      stage_factor(ck.j);
      if (rotate && threadIdx.x < (r >> 1))
        reinterpret_cast<float2*>(sph2)[threadIdx.x] =
            phase_of(om, pair_delta(cm, ck, threadIdx.x));
      __syncthreads();
      if constexpr (NT > 1) {
        switch (rotate ? hx : 0) {
          case 1: patch_tiles_batch<Q, MK, M8, PAGED, 1, OUT, NT>(c, cm, sV, sph2, s1, TB); break;
          case 2: patch_tiles_batch<Q, MK, M8, PAGED, 2, OUT, NT>(c, cm, sV, sph2, s1, TB); break;
          case 4: patch_tiles_batch<Q, MK, M8, PAGED, 4, OUT, NT>(c, cm, sV, sph2, s1, TB); break;
          case 8: patch_tiles_batch<Q, MK, M8, PAGED, 8, OUT, NT>(c, cm, sV, sph2, s1, TB); break;
          case -1: patch_tiles_batch<Q, MK, M8, PAGED, -1, OUT, NT>(c, cm, sV, sph2, s1, TB); break;
          default: patch_tiles_batch<Q, MK, M8, PAGED, 0, OUT, NT>(c, cm, sV, sph2, s1, TB); break;
        }
      } else {
        KAMERA_PATCH_SWITCH(true)
      }
    }
  } else {
    // The remaining chunks of the group, one after the other.
    int64_t t0 = start;
    ChunkRef ck = find_chunk_wave(cm, t0, from);
    bool staged = false;
    while (true) {
      const int64_t s1 = min(c.t1, ck.end);
      if (s1 > t0) {
        const bool rotate = r > 0 && ck.delta != 0;
        if (staged) __syncthreads();  // LDS still read by the previous chunk's tiles
        staged = true;
        stage(ck, rotate);
        __syncthreads();
        KAMERA_PATCH_SWITCH(false)
      }
      t0 = max(t0, s1);
      if (t0 >= c.t1 || ck.j + 1 >= cm.num_chunks) break;
      ck = find_chunk_wave(cm, t0, ck.j + 1);
    }
  }
#undef KAMERA_PATCH_SWITCH
}
#undef KAMERA_CH

// ------------------------------------------------------------------ generic rows

template <typename T>
__device__ __forceinline__ float dot_patch(const T* u, const T* v, int m) {
  float s = 0.f;
  for (int k = 0; k < m; ++k) s = fmaf(load_f(u + k), load_f(v + k), s);
  return s;
}

// Slot offset of token t in one layer of a (possibly paged) channel; false when its
// page id is out of range.
__device__ __forceinline__ bool slot_of(int64_t t, int page_size, const int32_t* table,
                                        int64_t num_pages, int64_t page_stride,
                                        int64_t slot_stride, int64_t* so) {
  if (page_size > 0) {
    const int64_t pg = table[t / page_size];
    *so = pg * page_stride + (t % page_size) * slot_stride;
    return pg >= 0 && pg < num_pages;
  }
  *so = t * slot_stride;
  return true;
}

template <typename T>
__device__ __forceinline__ void copy_bits(T* dst, const T* src) {
  if constexpr (sizeof(T) == 1) *(uint8_t*)dst = *(const uint8_t*)src;
  else if constexpr (sizeof(T) == 2) *(uint16_t*)dst = *(const uint16_t*)src;
  else *(uint32_t*)dst = *(const uint32_t*)src;
}

// One thread per (layer, token, head) row; any dim, any even rope_dim, any rank.
// OUT: the row is read through the channel's layout and written through its
// destination layout, whole (elements the call leaves alone are copied bit for bit).
// T = uint8_t: fp8 E4M3 codes of values scale * code, with bf16 factors.
template <typename T, bool OUT>
__global__ __launch_bounds__(kBlock) void generic_rows(ChanArgs ch, CommonArgs cm) {
  using FT = std::conditional_t<sizeof(T) == 1, uint16_t, T>;  // factor type
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
    const int64_t moves = chunk_moves(cm, j);
    if (!OUT && m == 0 && (moves == 0 || r == 0)) continue;
    int64_t so, dso = 0;
    if (!slot_of(t, cm.page_size, cm.block_table, cm.num_pages, ch.page_stride, ch.slot_stride,
                 &so))
      continue;
    if (OUT && !slot_of(t, cm.out_page_size, cm.out_block_table, cm.out_num_pages,
                        ch.out_page_stride, ch.out_slot_stride, &dso))
      continue;
    const T* src = (const T*)ch.data + layer * ch.layer_stride + so + h * ch.head_stride;
    T* dst = OUT ? (T*)ch.out + layer * ch.out_layer_stride + dso + h * ch.out_head_stride
                 : (T*)src;
    if (OUT && m == 0 && (moves == 0 || r == 0)) {
      for (int d = 0; d < D; ++d) copy_bits(dst + d, src + d);
      continue;
    }
    const FT* u = (const FT*)ch.U + (layer * Tt + t) * m;
    const FT* vr = (const FT*)ch.V + ((layer * cm.num_chunks + j) * F + h * D) * m;
    const float qs = sizeof(T) == 1 ? ch.scale[layer] : 1.f;
    const float qinv = sizeof(T) == 1 ? 1.f / qs : 1.f;
    for (int i = 0; i < half; ++i) {
      const int d0 = cm.pairing == 1 ? 2 * i : i;
      const int d1 = cm.pairing == 1 ? 2 * i + 1 : i + half;
      const int64_t di = cm.num_sections > 1
                             ? cm.delta[(int64_t)j * cm.num_sections + section_of(cm, i)]
                             : moves;
      if (di == 0 && m == 0) {  // this pair does not move
        if (OUT) {
          copy_bits(dst + d0, src + d0);
          copy_bits(dst + d1, src + d1);
        }
        continue;
      }
      float a = load_f(src + d0) * qs, b = load_f(src + d1) * qs;
      if (di != 0) {
        float c, s;
        phase_generic(cm.theta, r, i, di, c, s);
        const float an = fmaf(a, c, -(b * s));
        const float bn = fmaf(b, c, a * s);
        a = an;
        b = bn;
      }
      if (m > 0) {
        a += dot_patch(u, vr + (int64_t)d0 * m, m);
        b += dot_patch(u, vr + (int64_t)d1 * m, m);
      }
      store_f(dst + d0, a * qinv);
      store_f(dst + d1, b * qinv);
    }
    if (m > 0)
      for (int d = r; d < D; ++d)
        store_f(dst + d, (load_f(src + d) * qs + dot_patch(u, vr + (int64_t)d * m, m)) * qinv);
    else if (OUT)
      for (int d = r; d < D; ++d) copy_bits(dst + d, src + d);
  }
}

// ------------------------------------------------------------------ block-table inverse

__global__ __launch_bounds__(kBlock) void table_inverse_fill(int32_t* inv, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock)
    inv[i] = -1;
}

__global__ __launch_bounds__(kBlock) void table_inverse_scatter(const int32_t* table,
                                                                int64_t entries,
                                                                int64_t num_pages,
                                                                int32_t* inv) {
  for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < entries;
       k += (int64_t)gridDim.x * kBlock) {
    const int32_t pg = table[k];
    if (pg >= 0 && pg < num_pages) inv[pg] = (int32_t)k;
  }
}

// ------------------------------------------------------------------ library-held scratch

// The inverse block table of the no-allocation entry point: one array per GPU the
// library runs on, kept until the process ends.  Host code never names it except to look
// its address up (scratch_inverse_table); kernels get that address as an argument.
static __device__ __align__(256) int32_t scratch[kScratchPoolPages];

}  // namespace

// ------------------------------------------------------------------ library-held scratch

hipError_t scratch_inverse_table(hipStream_t s, int32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  hipDevice_t dev = 0;
  hipError_t e = hipStreamGetDevice(s, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // Each GPU holds its own copy of the array; its address is looked up once, with that
    // GPU current.
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = static_cast<int32_t*>(addr[dev]);
  return hipSuccess;
}

// ------------------------------------------------------------------ launchers

hipError_t launch_table_inverse(const int32_t* table, int64_t entries, int64_t num_pages,
                                int32_t* inv, hipStream_t s) {
  auto grid = [](int64_t n) {
    int64_t b = (n + kBlock - 1) / kBlock;
    return dim3((unsigned)(b < 1 ? 1 : b > 4096 ? 4096 : b));
  };
  hipLaunchKernelGGL(table_inverse_fill, grid(num_pages), dim3(kBlock), 0, s, inv, num_pages);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || entries == 0) return e;
  hipLaunchKernelGGL(table_inverse_scatter, grid(entries), dim3(kBlock), 0, s, table, entries,
                     num_pages, inv);
  return hipGetLastError();
}

hipError_t launch_rotate_rows(const ChanArgs& ch, const CommonArgs& cm, int unroll,
                              hipStream_t s) {
  const int64_t blocks = (int64_t)cm.num_layers * cm.token_groups;
  const dim3 grid((unsigned)blocks);
  const bool il = cm.pairing == 1;
  const bool sec = cm.num_sections > 1;
  const bool q = cm.dtype == 2;
#define KAMERA_LAUNCH_ROT4(LPR, PG, IL, SC)                                                          \
  do {                                                                                               \
    if (q && unroll == 8) hipLaunchKernelGGL((rotate_rows<true, LPR, 8, PG, IL, SC>), grid, dim3(kBlock), 0, s, ch, cm); \
    else if (q) hipLaunchKernelGGL((rotate_rows<true, LPR, 4, PG, IL, SC>), grid, dim3(kBlock), 0, s, ch, cm); \
    else if (unroll == 2) hipLaunchKernelGGL((rotate_rows<false, LPR, 2, PG, IL, SC>), grid, dim3(kBlock), 0, s, ch, cm); \
    else hipLaunchKernelGGL((rotate_rows<false, LPR, 4, PG, IL, SC>), grid, dim3(kBlock), 0, s, ch, cm); \
  } while (0)
#define KAMERA_LAUNCH_ROT3(LPR, PG, IL)                 \
  do {                                                  \
    if (sec) KAMERA_LAUNCH_ROT4(LPR, PG, IL, true);     \
    else KAMERA_LAUNCH_ROT4(LPR, PG, IL, false);        \
  } while (0)
#define KAMERA_LAUNCH_ROT2(LPR, PG)                 \
  do {                                              \
    if (il) KAMERA_LAUNCH_ROT3(LPR, PG, true);      \
    else KAMERA_LAUNCH_ROT3(LPR, PG, false);        \
  } while (0)
#define KAMERA_LAUNCH_ROT(LPR)                                  \
  do {                                                          \
    if (cm.page_size > 0) KAMERA_LAUNCH_ROT2(LPR, true);       \
    else KAMERA_LAUNCH_ROT2(LPR, false);                        \
  } while (0)
  switch (ch.rope_dim) {
    case 16: KAMERA_LAUNCH_ROT(2); break;
    case 32: KAMERA_LAUNCH_ROT(4); break;
    case 64: KAMERA_LAUNCH_ROT(8); break;
    case 128: KAMERA_LAUNCH_ROT(16); break;
    default: return hipErrorInvalidValue;
  }
#undef KAMERA_LAUNCH_ROT
#undef KAMERA_LAUNCH_ROT2
#undef KAMERA_LAUNCH_ROT3
#undef KAMERA_LAUNCH_ROT4
  return hipGetLastError();
}

hipError_t launch_relocate_patch_rows(const ChanArgs* ch, int nch, const CommonArgs& cm_in,
                                      int valu, bool pool, hipStream_t s) {
  ChanArgs c0 = ch[0];
  ChanArgs c1 = nch > 1 ? ch[1] : ch[0];
  if (nch == 1) c1.blocks = 0;
  CommonArgs cm = cm_in;
  cm.tail_mode = 0;
  int64_t bpl = c0.blocks + c1.blocks;
  dim3 grid((unsigned)((int64_t)cm.num_layers * bpl));
  // XCD grouping by the larger feature-block count of the launch's channels: a token
  // group's blocks of that channel land on one XCD; a channel with one block per group
  // (MLA's k_rope beside c_KV) then gets runs of consecutive token groups per XCD.  The
  // numbering is a bijection for any group size.
  const int xg = nch == 1 ? c0.fblocks : (c0.fblocks > c1.fblocks ? c0.fblocks : c1.fblocks);
  const int mk = (cm.rank + 31) / 32;
  const bool m8 = cm.rank % 8 == 0;
  // Out of place (recall): 1 contiguous destination, 2 paged destination.
  const int out = c0.out == nullptr ? 0 : (cm.out_page_size > 0 ? 2 : 1);
  const bool q = cm.dtype == 2;
  if (out > 0 && (!m8 || (nch > 1 && c1.out == nullptr))) return hipErrorInvalidValue;
  if (out == 0 && mk == 0) return hipErrorInvalidValue;
  if (q && !m8) return hipErrorInvalidValue;
  if (pool) {
    if (out > 0 || mk == 0 || cm.num_chunks != 1 || cm.page_size <= 0 || cm.page_size % 16 != 0 ||
        cm.inv == nullptr)
      return hipErrorInvalidValue;
    // Tiles each wave requests together: its whole share when that is 2 tiles, or 3 of
    // fp8 (three bf16 tiles exceed the register budget of 3 waves per SIMD and spill).
    const int tpw = cm.block_tokens / 64;
    const int pool_nt = (tpw == 2 || (tpw == 3 && q)) && cm.block_tokens % 64 == 0 ? tpw : 1;
#define KAMERA_LAUNCH_POOL_NT(Q, MK, M8, NT)                                                  \
  hipLaunchKernelGGL((relocate_patch_rows<Q, MK, M8, true, false, 0, false, true, NT>), grid,   \
                     dim3(kBlock), 0, s, c0, c1, cm, bpl, xg)
#define KAMERA_LAUNCH_POOL(Q, MK, M8)                                    \
  do {                                                                   \
    if (pool_nt == 3) KAMERA_LAUNCH_POOL_NT(Q, MK, M8, (Q ? 3 : 1));     \
    else if (pool_nt == 2) KAMERA_LAUNCH_POOL_NT(Q, MK, M8, 2);          \
    else KAMERA_LAUNCH_POOL_NT(Q, MK, M8, 1);                            \
  } while (0)
    if (q && mk == 1) KAMERA_LAUNCH_POOL(true, 1, true);
    else if (q && mk == 2) KAMERA_LAUNCH_POOL(true, 2, true);
    else if (q && mk <= 4) KAMERA_LAUNCH_POOL(true, 4, true);
    else if (mk == 1) { if (m8) KAMERA_LAUNCH_POOL(false, 1, true); else KAMERA_LAUNCH_POOL(false, 1, false); }
    else if (mk == 2) { if (m8) KAMERA_LAUNCH_POOL(false, 2, true); else KAMERA_LAUNCH_POOL(false, 2, false); }
    else if (mk <= 4) { if (m8) KAMERA_LAUNCH_POOL(false, 4, true); else KAMERA_LAUNCH_POOL(false, 4, false); }
    else return hipErrorInvalidValue;
#undef KAMERA_LAUNCH_POOL
#undef KAMERA_LAUNCH_POOL_NT
    return hipGetLastError();
  }
#define KAMERA_LAUNCH_K(Q, MK, M8, PG, TL, OUT, XG)                                           \
  hipLaunchKernelGGL((relocate_patch_rows<Q, MK, M8, PG, TL, OUT>), grid, dim3(kBlock), 0, s, \
                     c0, c1, cm, bpl, XG)
#define KAMERA_LAUNCH_B2(Q, MK, M8, PG, XG, CHS)                                               \
  hipLaunchKernelGGL((relocate_patch_rows<Q, (MK > 2 ? 1 : MK), M8, PG, false, 0, false, false, \
                                          2, CHS>),                                             \
                     grid, dim3(kBlock), 0, s, c0, c1, cm, bpl, XG)
#define KAMERA_LAUNCH_B(Q, MK, M8, PG, XG)                                   \
  do {                                                                       \
    if (cm.num_chunks == 1) KAMERA_LAUNCH_B2(Q, MK, M8, PG, XG, 1);          \
    else KAMERA_LAUNCH_B2(Q, MK, M8, PG, XG, 2);                             \
  } while (0)
#define KAMERA_LAUNCH_IN(MK, PG, TL, XG)                                      \
  do {                                                                        \
    if (!TL && MK <= 2 && batch && q) KAMERA_LAUNCH_B(true, MK, true, PG, XG); \
    else if (!TL && MK <= 2 && batch && m8) KAMERA_LAUNCH_B(false, MK, true, PG, XG); \
    else if (!TL && MK <= 2 && batch) KAMERA_LAUNCH_B(false, MK, false, PG, XG); \
    else if (q) KAMERA_LAUNCH_K(true, MK, true, PG, TL, 0, XG);               \
    else if (m8 && valu && !TL && MK <= 2)                                    \
      hipLaunchKernelGGL((relocate_patch_rows<false, MK, true, PG, false, 0,  \
                                              (MK <= 2 && !TL)>),             \
                         grid, dim3(kBlock), 0, s, c0, c1, cm, bpl, XG);      \
    else if (m8) KAMERA_LAUNCH_K(false, MK, true, PG, TL, 0, XG);             \
    else KAMERA_LAUNCH_K(false, MK, false, PG, TL, 0, XG);                    \
  } while (0)
#define KAMERA_LAUNCH_OUT(MK, PG, TL, XG)                                     \
  do {                                                                        \
    if (q && out == 1) KAMERA_LAUNCH_K(true, MK, true, PG, TL, 1, XG);        \
    else if (q) KAMERA_LAUNCH_K(true, MK, true, PG, TL, 2, XG);               \
    else if (out == 1) KAMERA_LAUNCH_K(false, MK, true, PG, TL, 1, XG);       \
    else KAMERA_LAUNCH_K(false, MK, true, PG, TL, 2, XG);                     \
  } while (0)
#define KAMERA_LAUNCH_PG(MK, TL, XG)                                          \
  do {                                                                        \
    if (out > 0) {                                                            \
      if (cm.page_size > 0) KAMERA_LAUNCH_OUT(MK, true, TL, XG);              \
      else KAMERA_LAUNCH_OUT(MK, false, TL, XG);                              \
    } else {                                                                  \
      if (cm.page_size > 0) KAMERA_LAUNCH_IN(MK, true, TL, XG);               \
      else KAMERA_LAUNCH_IN(MK, false, TL, XG);                               \
    }                                                                         \
  } while (0)
#define KAMERA_LAUNCH_MK(TL, XG)                                              \
  do {                                                                        \
    if (mk == 0) {                                                            \
      if (cm.page_size > 0) KAMERA_LAUNCH_OUT(0, true, TL, XG);               \
      else KAMERA_LAUNCH_OUT(0, false, TL, XG);                               \
    } else if (mk == 1) KAMERA_LAUNCH_PG(1, TL, XG);                          \
    else if (mk == 2) KAMERA_LAUNCH_PG(2, TL, XG);                            \
    else if (mk <= 4) KAMERA_LAUNCH_PG(4, TL, XG);                            \
    else return hipErrorInvalidValue;                                         \
  } while (0)
  // In place, at least two tiles per wave: each wave of the head launch requests its first
  // two tiles together (two tiles in flight per wave).
  bool batch = out == 0 && !valu && cm.block_tokens >= 128;
  // Groups that a chunk boundary cuts.  In place, with no more boundaries than groups,
  // the head launch takes one unit per boundary after its token groups (each covers one
  // chunk's part of a cut group), so one launch covers the call.  Otherwise a second
  // launch walks the cut groups chunk by chunk, indexed by boundary (out of place:
  // the boundary units would raise the head kernel's register count past 128) or, when
  // boundaries outnumber groups, by group.
  const int64_t nb = (int64_t)cm.num_chunks - 1;
  const bool fold = out == 0 && nb > 0 && nb <= cm.token_groups;
  if (fold) {
    c0.blocks += nb * c0.fblocks;
    if (nch > 1) c1.blocks += nb * c1.fblocks;
    bpl = c0.blocks + c1.blocks;
    grid = dim3((unsigned)((int64_t)cm.num_layers * bpl));
  }
  KAMERA_LAUNCH_MK(false, xg);
  batch = false;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || cm.num_chunks < 2 || fold) return e;
  cm.tail_mode = nb <= cm.token_groups ? 1 : 2;
  const int64_t units = cm.tail_mode == 1 ? nb : cm.token_groups;
  c0.blocks = units * c0.fblocks;
  c1.blocks = nch > 1 ? units * c1.fblocks : 0;
  bpl = c0.blocks + c1.blocks;
  grid = dim3((unsigned)((int64_t)cm.num_layers * bpl));
  KAMERA_LAUNCH_MK(true, 0);
#undef KAMERA_LAUNCH_MK
#undef KAMERA_LAUNCH_B
#undef KAMERA_LAUNCH_B2
#undef KAMERA_LAUNCH_PG
#undef KAMERA_LAUNCH_OUT
#undef KAMERA_LAUNCH_IN
#undef KAMERA_LAUNCH_K
  return hipGetLastError();
}

hipError_t launch_generic(const ChanArgs& ch, const CommonArgs& cm, int dtype, hipStream_t s) {
  const int64_t nrows = (int64_t)cm.num_layers * cm.total_tokens * ch.heads;
  int64_t blocks = (nrows + kBlock - 1) / kBlock;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  const bool out = ch.out != nullptr;
  if (dtype == 2 && out)
    hipLaunchKernelGGL((generic_rows<uint8_t, true>), dim3((unsigned)blocks), dim3(kBlock), 0, s, ch, cm);
  else if (dtype == 2)
    hipLaunchKernelGGL((generic_rows<uint8_t, false>), dim3((unsigned)blocks), dim3(kBlock), 0, s, ch, cm);
  else if (dtype == 0 && out)
    hipLaunchKernelGGL((generic_rows<uint16_t, true>), dim3((unsigned)blocks), dim3(kBlock), 0, s, ch, cm);
  else if (dtype == 0)
    hipLaunchKernelGGL((generic_rows<uint16_t, false>), dim3((unsigned)blocks), dim3(kBlock), 0, s, ch, cm);
  else if (out)
    hipLaunchKernelGGL((generic_rows<float, true>), dim3((unsigned)blocks), dim3(kBlock), 0, s, ch, cm);
  else
    hipLaunchKernelGGL((generic_rows<float, false>), dim3((unsigned)blocks), dim3(kBlock), 0, s, ch, cm);
  return hipGetLastError();
}

}  // namespace kamera
