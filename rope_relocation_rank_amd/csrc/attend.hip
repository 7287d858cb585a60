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
//                 transposed from the wave's LDS tile, which the V and U_V rows reach
//                 straight from memory (no registers), one tile ahead.  Each (range,
//                 chunk) segment writes one partial: max, sum, the 128 value sums and
//                 the m U_V sums.
//   attend_merge  per (layer, query head): merges the partials, adding V_V times each
//                 partial's U_V sums with that partial's chunk factor.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kamera_internal.h"
#include "rope_device.h"

namespace kamera {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef int v2i32_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;      // prep and tile kernels
constexpr int kD = kAttendDim;

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
// each query head's rotated query and V_K^T q.  The V_K rows take 256 rank bytes of
// dynamic LDS, so that small ranks leave room for more workgroups per CU (each one
// waits on two rounds of loads).
__global__ __launch_bounds__(kThreads) void attend_prep(AttendArgs a) {
  extern __shared__ __align__(16) uint16_t svk[];  // V_K[g * 128 + d][k], kD * rank
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
  // fp8 keys are scale * code: the rotated query carries K's scale of the layer, so the
  // tile kernel multiplies codes by it.
  const float kscale = a.scale_log2 * (a.kv_scale[0] ? a.kv_scale[0][l] : 1.f);
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
    out[(int64_t)h * W + d] = v * kscale;
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

// Buffer addressing (gfx9 raw buffer, stride 0): a resource covers `bytes` bytes from a
// wave-uniform base and range-checks every access, so a load at byte offset kOob reads
// zeros; rows a lane skips take that offset instead of a branch.  The offset passes an
// empty asm operand so that the compiler does not split the access into branches (a
// load behind such a branch waits for every earlier load).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
// 16 bytes into registers (aux 2: nontemporal, for rows read once).
template <int AUX>
__device__ __forceinline__ u32x4_t bload(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)opaque(off), 0, AUX);
}
// Waits until at most n vector-memory requests of this wave are outstanding (vmcnt;
// the export and LDS counters are left alone).
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}
// 16 bytes per lane straight into LDS: lane i's bytes land at dst + 16 i (dst is
// wave-uniform).  No registers are held while the request is in flight.  The compiler
// does not reliably wait for these before later LDS reads of the same bytes, so the
// tile loop waits for them itself (wait_vm), with the requests kept in program order.
__device__ __forceinline__ void bload_lds(rsrc_t r, uint32_t off, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           (int)opaque(off), 0, 0, 2);
}

// 8-byte loads and fp8 E4M3 codes.  Every E4M3 value is a bf16 value (3 mantissa bits),
// so a code becomes bf16 exactly: to fp32 by the hardware conversion, then the upper
// half of the fp32 pattern (NaN stays NaN).
template <int AUX>
__device__ __forceinline__ u32x2_t bload8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)opaque(off), 0, AUX);
}
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  const f32x2_t v = hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
                       : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  return (__float_as_uint(v[0]) >> 16) | (__float_as_uint(v[1]) & 0xffff0000u);
}
__device__ __forceinline__ u32x4_t fp8x8_to_bf16x8(u32x2_t w) {
  return u32x4_t{fp8x2_to_bf16x2(w[0], false), fp8x2_to_bf16x2(w[0], true),
                 fp8x2_to_bf16x2(w[1], false), fp8x2_to_bf16x2(w[1], true)};
}
__device__ __forceinline__ uint16_t fp8_to_bf16(uint32_t code) {
  return (uint16_t)(__float_as_uint(__builtin_amdgcn_cvt_f32_fp8((int)code, 0)) >> 16);
}

// One wave's LDS tile: the V rows of its 16 tokens as four blocks of four 256-byte rows
// (token 4 b + i in block b, row i), the blocks padded so that the reads of the four
// lane groups fall in different banks (the kernel's kVB: 64 bytes for per-element reads,
// 128 with transposing reads); and, in an array of its own, the U_V rows of the 16
// tokens as they lie in memory (16 x 2m bytes, m <= 32 MK).  Separate arrays let the
// compiler wait for exactly the request a read depends on.
// fp8 (rows of 128 bytes): two blocks of eight rows (token 8 b + i in block b, row i).
constexpr int kVBlkQ = 8 * kD + 64;
constexpr int kVTileQ = 2 * kVBlkQ;

// The K-side rows of one tile as loaded: lane (c16, grp) holds features 32 ks + 8 grp ..
// + 7 of token c16 (k), and ranks 32 ku + 8 grp .. + 7 of its U_K row (uk).
template <int MKX, bool Q>
struct KRows {
  u32x4_t k[Q ? 1 : 4], uk[MKX];
  u32x2_t k8[Q ? 4 : 1];  // fp8: 8 codes per step, converted when used
};
// Where the lane's token of a tile lives: byte offsets of its K and V rows inside the
// layer (kOob when the token lies past the segment or its page is out of range).
struct RowAt {
  uint32_t k, v;
};
// Block-table entries of one tile with pages of at least 16 slots: the tile's tokens
// lie in at most two pages, entries p0 (of its first token) and p1 (of its last), and
// its first token sits at slot r0 of the first page.  Wave-uniform: scalar loads.
struct TilePages {
  int32_t p0, p1, r0;
};

// One 4-wave workgroup per (layer, KV head, token range); the waves take the range's
// 16-token tiles w, w + 4, ... and merge through LDS at the end of each segment (the
// part of the range inside one chunk), which writes one partial slot per query head.
// The query-side B operands (high and low parts of the rotated query and of V_K^T q)
// are the same for the four waves and sit once in LDS.  Per tile, a wave requests the
// K and U_K rows into registers and the V and U_V rows straight into its LDS tile (the
// P V products read them transposed from there), one tile ahead of the one it works
// on: DB, the next tile's V and U_V go to a second LDS tile at once; otherwise they go
// to the one LDS tile after the current tile's reads.  Block-table entries are read two
// tiles ahead, before the rows that precede their use, so no wait for them waits for
// rows.  MK: 32-wide rank steps (ceil(m / 32)).  PG: 0 contiguous; 1 paged with pages
// of at least 16 slots, a tile's two block-table entries read by scalar loads (which
// count apart from the row requests); 2 paged with smaller pages, each lane reading its
// token's entry.
// Q: fp8 E4M3 keys and values (per-layer scales); K rows are converted to bf16 in
// registers, V rows read from LDS as codes.  HM: one workgroup per (layer, token
// range) with one wave per KV head (heads <= 8), each wave walking every tile of the
// range and writing its own partials; the waves request the same U rows at about the
// same time from one CU, so those are fetched once per range instead of once per head.
template <int MK, int PG, bool DB, bool Q, bool HM>
__global__ __launch_bounds__(HM ? 64 * kAttendMaxHeadsPerGroup : kThreads)
__attribute__((amdgpu_waves_per_eu(MK >= 4 && DB ? 1 : MK >= 2 || HM ? 2 : 3)))
void attend_tiles(AttendArgs a) {
  constexpr int MKX = MK > 0 ? MK : 1;
  constexpr int NW = HM ? kAttendMaxHeadsPerGroup : kWaves;  // waves per workgroup (at most)
  constexpr int TSTEP = HM ? 1 : kWaves;                      // a wave's tile stride
  constexpr uint32_t ES = Q ? 1 : 2;  // bytes per KV element
  constexpr int kVT = Q ? kVTileQ : 4 * (4 * 2 * kD + (MK <= 1 ? 128 : 64));
  constexpr int MU = 2 * MK;  // 16-wide rank blocks of the U_V sums
  // fp8 V codes through transposing LDS reads: measured faster with one 32-rank step
  // (Qwen-shaped fp8 call 0.0615 -> 0.0587 ms) and slower with two (72B-shaped fp8 call
  // 1.630 -> 1.671 ms, double-buffered tiles).
  constexpr bool kTr8 = Q && MK <= 1;
  // bf16 with one 32-rank step: V through the transposing 16-bit LDS read, rows' 32-byte
  // slots XOR-placed by row and blocks 128 bytes apart (64 for the per-element reads).
  constexpr bool kTr16 = !Q && MK <= 1;
  constexpr int kVB = 4 * 2 * kD + (kTr16 ? 128 : 64);
  constexpr int MUX = MU > 0 ? MU : 1;
  constexpr int kUTile = 1024 * MKX;
  constexpr int kMergeBytes = HM ? 0 : kWaves * kAttendMaxGroup * (2 + kD + 32 * MK) * 4;
  constexpr int kBuf0 = NW * kVT > kMergeBytes ? NW * kVT : kMergeBytes;
  constexpr int kBOps = 8 + 2 * MKX;  // 16-byte query-side operands per lane
  __shared__ __align__(16) unsigned char lds0[kBuf0];  // V tiles, then the merge
  __shared__ __align__(16) unsigned char lds1[DB ? NW * kVT : 16];
  __shared__ __align__(16) unsigned char ldu0[NW * kUTile];  // U_V tiles
  __shared__ __align__(16) unsigned char ldu1[DB ? NW * kUTile : 16];
  __shared__ __align__(16) u32x4_t sB[HM ? 1 : kBOps * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;
  const int grp = lane >> 4;
  // LDS tiles are addressed as one byte offset into the array itself (buffer 0 or 1, a
  // compile-time tag), so that the compiler keeps track of which array every read and
  // every request touches and waits for exactly the requests a read depends on.
  using Buf0 = std::integral_constant<int, 0>;
  using Buf1 = std::integral_constant<int, 1>;
  const int vwave = wave * kVT, uwave = wave * kUTile;
  typedef float MergeRow[kAttendMaxGroup][2 + kD + 32 * MK];
  MergeRow* sred = (MergeRow*)lds0;

  const uint32_t S = (uint32_t)a.splits;
  const uint32_t H = (uint32_t)a.heads;
  const uint32_t bid = blockIdx.x;
  int s, l, g;
  if constexpr (HM) {
    // Split fastest, then layer; wave w runs KV head w.
    l = (int)(bid / S);
    s = (int)(bid - (uint32_t)l * S);
    g = wave;
  } else {
    // Split fastest, then KV head, then layer.  (Placing the KV heads of one (layer,
    // split) on one XCD, so that they read the range's U rows from one L2, measured 3-4%
    // slower.)
    const uint32_t lg = bid / S;
    s = (int)(bid - lg * S);
    l = (int)(lg / H);
    g = (int)(lg - (uint32_t)l * H);
  }
  const int64_t T = a.total_tokens;
  const int64_t t_lo = (int64_t)s * a.split_tokens;
  const int64_t t_hi = min(T, t_lo + (int64_t)a.split_tokens);
  if (t_lo >= t_hi) return;
  const int m = a.rank, gq = a.group, Hq = a.num_q_heads, n = a.num_chunks;
  const int W = kD + m;
  const bool hv = c16 < gq;  // this lane's MFMA column is a real query head
  const uint32_t ss0 = (uint32_t)a.slot_stride[0] * ES, ss1 = (uint32_t)a.slot_stride[1] * ES;
  const uint32_t ps0 = (uint32_t)a.page_stride[0] * ES, ps1 = (uint32_t)a.page_stride[1] * ES;
  // fp8: the value sums are sums of p * code; V's scale of the layer turns them into
  // values when the partial is written.
  const float vscale = Q ? a.kv_scale[1][l] : 1.f;
  const uint32_t P = (uint32_t)a.page_size;
  const int psh = (P != 0u && (P & (P - 1u)) == 0u) ? __builtin_ctz(P) : -1;
  // One resource per (layer, head) row set, from the head's first element to the end of
  // the layer; one per layer of each U factor; one over the block table.
  const rsrc_t rk = make_rsrc((const unsigned char*)a.data[0] +
                                  ((int64_t)l * a.layer_stride[0] + (int64_t)g * a.head_stride[0]) * ES,
                              a.layer_bytes[0] - (uint32_t)(g * a.head_stride[0] * ES));
  const rsrc_t rv = make_rsrc((const unsigned char*)a.data[1] +
                                  ((int64_t)l * a.layer_stride[1] + (int64_t)g * a.head_stride[1]) * ES,
                              a.layer_bytes[1] - (uint32_t)(g * a.head_stride[1] * ES));
  const uint32_t ubytes = (uint32_t)(T * m * 2);
  const rsrc_t ruk = make_rsrc(MK > 0 ? (const void*)((const uint16_t*)a.U[0] + (int64_t)l * T * m)
                                      : (const void*)a.q, MK > 0 ? ubytes : 0u);
  const rsrc_t ruv = make_rsrc(MK > 0 ? (const void*)((const uint16_t*)a.U[1] + (int64_t)l * T * m)
                                      : (const void*)a.q, MK > 0 ? ubytes : 0u);
  const rsrc_t rbt = make_rsrc(PG == 2 ? (const void*)a.block_table : (const void*)a.q,
                               PG == 2 ? (uint32_t)(((T + P - 1) / P) * 4) : 0u);
  // Restricted copies: the slot stores cannot clobber the table, so uniform reads of it
  // become scalar loads.
  const int32_t* __restrict__ bt = a.block_table;
  float* __restrict__ wsp = a.ws;

  for (int64_t t0 = t_lo; t0 < t_hi;) {
    const int j = chunk_at(a.offsets, n, t0);
    const int64_t s1 = min(t_hi, a.offsets[j + 1]);
    if (s1 <= t0) break;  // offsets that do not cover the range: nothing more here
    const int ntiles = (int)((s1 - t0 + 15) >> 4);

    // HM: the wave applies V_V of the segment's chunk to its U_V sums itself (then the
    // merge has no per-chunk work).  Lane (c16, grp) takes, for each 16-feature block fb
    // and 16-rank block ub, ranks 16 ub + 4 grp .. + 3 of V_V row 16 fb + c16: the A
    // operand of a 16x16x16 product whose B operand is uacc[ub] as the lane holds it.
    // With one 32-rank step, ranks 0 .. 15 are requested here, to arrive during the
    // tiles (ranks 16 .. 31, if m has them, in the epilogue); ranks past m read the
    // row's start and count zero.
    const uint16_t* vvseg = (const uint16_t*)a.V[1] + (((int64_t)l * n + j) * H + g) * kD * m;
    auto vv_load = [&](int fb, int ub) -> u32x2_t {
      const int k0 = 16 * ub + 4 * grp;
      const u32x2_t w = *(const u32x2_t*)(vvseg + (16 * fb + c16) * m + (k0 < m ? k0 : 0));
      return k0 < m ? w : u32x2_t{0u, 0u};
    };
    constexpr bool kVVPre = HM && MK == 1;
    u32x2_t vvr[kVVPre ? 8 : 1];
    if constexpr (kVVPre) {
#pragma unroll
      for (int fb = 0; fb < 8; ++fb) vvr[fb] = vv_load(fb, 0);
    }

    // Page lookups of tile ti: PG 1, the tile's two entries (uniform); PG 2, the entry
    // of the lane's token (-1: past the segment or out of the pool); PG 0, none.
    auto lookup = [&](int ti) {
      if constexpr (PG == 1) {
        // Tiles past the segment read the entries of its last token (their rows are
        // dropped anyway): no branch around the loads.
        TilePages q;
        const int64_t tb = t0 + 16 * (int64_t)ti;
        const uint32_t tt = (uint32_t)min(tb, s1 - 1), last = (uint32_t)(min(s1, tb + 16) - 1);
        const uint32_t i0 = psh >= 0 ? tt >> psh : tt / P;
        const uint32_t i1 = psh >= 0 ? last >> psh : last / P;
        q.r0 = (int32_t)(tt - i0 * P);
        q.p0 = bt[__builtin_amdgcn_readfirstlane(i0)];
        q.p1 = bt[__builtin_amdgcn_readfirstlane(i1)];
        return q;
      } else if constexpr (PG == 2) {
        const int64_t t = t0 + 16 * (int64_t)ti + c16;
        const uint32_t tt = (uint32_t)t;
        const uint32_t off = t < s1 ? (psh >= 0 ? tt >> psh : tt / P) * 4u : kOob;
        const int32_t pg = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rbt, (int)opaque(off), 0, 0);
        return (off == kOob || pg < 0 || pg >= a.num_pages) ? (int32_t)-1 : pg;
      } else {
        return 0;
      }
    };
    using Pages = decltype(lookup(0));
    auto row_at = [&](int ti, const Pages& pq) -> RowAt {
      const int64_t t = t0 + 16 * (int64_t)ti + c16;
      const uint32_t tt = (uint32_t)t;
      RowAt r{kOob, kOob};
      if constexpr (PG == 1) {
        const int32_t rr = pq.r0 + c16;
        const bool second = rr >= (int32_t)P;
        const int32_t pg = second ? pq.p1 : pq.p0;
        const uint32_t si = (uint32_t)(second ? rr - (int32_t)P : rr);
        const bool ok = t < s1 && pg >= 0 && pg < a.num_pages;
        r.k = ok ? (uint32_t)pg * ps0 + si * ss0 : kOob;
        r.v = ok ? (uint32_t)pg * ps1 + si * ss1 : kOob;
      } else if constexpr (PG == 2) {
        const uint32_t pi = psh >= 0 ? tt >> psh : tt / P, si = tt - pi * P;
        const bool ok = t < s1 && pq >= 0;
        r.k = ok ? (uint32_t)pq * ps0 + si * ss0 : kOob;
        r.v = ok ? (uint32_t)pq * ps1 + si * ss1 : kOob;
      } else {
        r.k = t < s1 ? tt * ss0 : kOob;
        r.v = t < s1 ? tt * ss1 : kOob;
      }
      return r;
    };
    // K and U_K rows of tile ti into registers.
    auto issue_k = [&](int ti, const RowAt& r, KRows<MKX, Q>& R) {
      const uint32_t tt = (uint32_t)(t0 + 16 * (int64_t)ti + c16);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint32_t off = r.k == kOob ? kOob : r.k + ES * (32u * ks + 8u * grp);
        if constexpr (Q) R.k8[ks] = bload8<2>(rk, off);
        else R.k[ks] = bload<2>(rk, off);
      }
#pragma unroll
      for (int ku = 0; ku < MKX; ++ku) {
        const int k0 = 32 * ku + 8 * grp;
        R.uk[ku] = u32x4_t{0u, 0u, 0u, 0u};
        if (MK > 0) R.uk[ku] = bload<0>(ruk, k0 < m ? (tt * (uint32_t)m + k0) * 2u : kOob);
      }
    };
    // V and U_V rows of tile ti straight into an LDS tile: request b copies tokens
    // 4 b .. 4 b + 3 (lane i: token 4 b + i / 16, bytes 16 (i % 16) of its row, whose
    // offset the lane of that token holds); the U_V rows of the 16 tokens are one
    // contiguous run of 32 m bytes, copied 1 KB per request (tokens past the segment
    // read zeros).
    auto issue_v = [&](int ti, const RowAt& r, auto buf) {
      constexpr bool one = decltype(buf)::value == 1;
      if constexpr (Q) {
        // tokens 8 b + lane / 8; with transposing reads (kTr8) row i of a block holds the
        // row's 16-byte chunk q at place q ^ ((i >> 1) & 3), so that the reads of the
        // eight rows of a block fall in different banks.
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const uint32_t vr = (uint32_t)__shfl((int)r.v, 8 * b + (lane >> 3));
          const uint32_t q16 = kTr8 ? (uint32_t)((lane & 7) ^ ((lane >> 4) & 3)) : (uint32_t)(lane & 7);
          bload_lds(rv, vr == kOob ? kOob : vr + 16u * q16,
                    one ? lds1 + (vwave + b * kVBlkQ) : lds0 + (vwave + b * kVBlkQ));
        }
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t vr = (uint32_t)__shfl((int)r.v, 4 * b + grp);
          // kTr16: row grp of the block holds the row's 16-byte chunk q at q ^ 2 grp
          const uint32_t q16 = kTr16 ? (uint32_t)(c16 ^ (2 * grp)) : (uint32_t)c16;
          bload_lds(rv, vr == kOob ? kOob : vr + 16u * q16,
                    one ? lds1 + (vwave + b * kVB) : lds0 + (vwave + b * kVB));
        }
      }
      const int64_t tb = t0 + 16 * (int64_t)ti;
#pragma unroll
      for (int b = 0; b < MK; ++b) {
        const int u = 64 * b + lane;  // 16-byte unit of the run; token tb + 8 u / m
        const bool ok = u < 2 * m && tb + (8 * u) / m < s1;
        bload_lds(ruv, ok ? (uint32_t)(tb * m * 2) + 16u * u : kOob,
                  one ? ldu1 + (uwave + 1024 * b) : ldu0 + (uwave + 1024 * b));
      }
    };

    // B operands: this lane's query head (column c16), features 32 ks + 8 grp ...  HM:
    // in registers (each wave its own head).  Otherwise every wave writes the same values
    // to LDS for the segment; the previous segment's readers all passed the barrier that
    // ends it.
    bf16x8_t bq[HM ? kBOps : 1];
    {
      const float* qp = a.qw + (((int64_t)l * n + j) * Hq + g * gq + (hv ? c16 : 0)) * W;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = hv ? qp[32 * ks + 8 * grp + e] : 0.f;
        bf16x8_t hi, lo;
        split8(x, hi, lo);
        if constexpr (HM) {
          bq[ks] = hi;
          bq[4 + ks] = lo;
        } else {
          sB[ks * 64 + lane] = __builtin_bit_cast(u32x4_t, hi);
          sB[(4 + ks) * 64 + lane] = __builtin_bit_cast(u32x4_t, lo);
        }
      }
#pragma unroll
      for (int ku = 0; ku < MKX; ++ku) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = 32 * ku + 8 * grp + e;
          x[e] = (MK > 0 && hv && k < m) ? qp[kD + k] : 0.f;
        }
        bf16x8_t hi, lo;
        split8(x, hi, lo);
        if constexpr (HM) {
          bq[8 + ku] = hi;
          bq[8 + MKX + ku] = lo;
        } else {
          sB[(8 + ku) * 64 + lane] = __builtin_bit_cast(u32x4_t, hi);
          sB[(8 + MKX + ku) * 64 + lane] = __builtin_bit_cast(u32x4_t, lo);
        }
      }
    }
    auto bop = [&](int o) -> bf16x8_t {
      if constexpr (HM) return bq[o];
      else return __builtin_bit_cast(bf16x8_t, sB[o * 64 + lane]);
    };

    float mrun = -INFINITY, lrun = 0.f;
    f32x4_t acc[8], uacc[MUX];
#pragma unroll
    for (int f = 0; f < 8; ++f) acc[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < MUX; ++u) uacc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Scores, online softmax and the P V and P U_V products of tile ti.
    // Requests per tile: K and U_K rows into registers, V and U_V rows into LDS, and
    // with small pages one block-table read per lane.
    constexpr int kReqK = 4 + MK, kReqV = (Q ? 2 : 4) + MK, kReqPg = PG == 2 ? 1 : 0;
    auto work = [&](const RowAt& r, const KRows<MKX, Q>& R, auto buf) {
      constexpr bool one = decltype(buf)::value == 1;
      const unsigned char* vs = one ? lds1 : lds0;
      const unsigned char* us = one ? ldu1 : ldu0;
      // Scores of tokens tb + 4 grp + i (i < 4) for query head c16.
      f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x4_t kw;
        if constexpr (Q) kw = fp8x8_to_bf16x8(R.k8[ks]);
        else kw = R.k[ks];
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, kw);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bop(ks), sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bop(4 + ks), sc, 0, 0, 0);
      }
#pragma unroll
      for (int ku = 0; ku < MK; ++ku) {
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, R.uk[ku]);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bop(8 + ku), sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bop(8 + MKX + ku), sc, 0, 0, 0);
      }
      // Tokens without a row (past the segment, or out of the pool) get weight 0: bit
      // c16 of the ballot over lanes 0..15 says whether token tb + c16 has one.
      const uint32_t onm = (uint32_t)__ballot(r.k != kOob) & 0xffffu;
      float s4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) s4[i] = (onm >> (4 * grp + i)) & 1u ? sc[i] : -INFINITY;
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
      // O^T[f][h] += V^T[f][t] P^T[t][h]: A = V^T rows f = 16 fb + c16, tokens 4 grp + i
      // (block grp, row i of the LDS tile).
      // This tile's V and U_V requests are done once no more than the requests issued
      // after them are outstanding: the next tile's block-table read, K and U_K rows
      // and (DB) V and U_V rows.
      wait_vm<kReqPg + kReqK + (DB ? kReqV : 0)>();
      __builtin_amdgcn_sched_barrier(0);
      // bf16: token 4 grp + i is row i of block grp; fp8: row 4 (grp % 2) + i of block
      // grp / 2.  kTr8 reads fp8 codes with the gfx950 transposing 8-bit LDS read: within
      // a 16-lane group, lane i receives as its byte e byte i & 7 of the 8 bytes lane
      // 2 e + (i >> 3) addressed.  Lane s addresses row 4 (grp % 2) + ((s >> 1) & 3)
      // (rows 4 .. 7 of the read repeat rows 0 .. 3) at features 16 fb + 8 (s & 1), so
      // lane c16 receives feature 16 fb + c16 of the group's four tokens in its low 4
      // bytes.  Otherwise one byte read per token.
      const int vrow = kTr8 ? 4 * (grp & 1) + ((c16 >> 1) & 3) : 4 * (grp & 1);
      // kTr16: the 16-bit transposing read gives lane i, as its element e, element i & 3
      // of the 8 bytes lane 4 e + (i >> 2) of its group addressed; lane s addresses row
      // s >> 2 of block grp at features 16 fb + 4 (s & 3), so lane c16 receives feature
      // 16 fb + c16 of the block's four tokens.
      const int vo = Q ? vwave + (grp >> 1) * kVBlkQ + vrow * kD + (kTr8 ? 8 * (c16 & 1) : c16)
                       : kTr16 ? vwave + grp * kVB + (c16 >> 2) * 2 * kD + 8 * (c16 & 3)
                               : vwave + grp * kVB + 2 * c16;
      const int vsw = (vrow >> 1) & 3;
#pragma unroll
      for (int fb = 0; fb < 8; ++fb) {
        bf16x4_t A;
        if constexpr (kTr8) {
          const uint32_t w = (uint32_t)__builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) v2i32_t*)(vs + vo + 16 * (fb ^ vsw)))[0];
          A = __builtin_bit_cast(bf16x4_t, u32x2_t{fp8x2_to_bf16x2(w, false), fp8x2_to_bf16x2(w, true)});
        } else if constexpr (Q) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            A[i] = __builtin_bit_cast(__bf16, fp8_to_bf16(vs[vo + i * kD + 16 * fb]));
        } else if constexpr (kTr16) {
          A = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) i16x4_t*)(vs + vo + 32 * (fb ^ (c16 >> 2)))));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            A[i] = __builtin_bit_cast(__bf16, *(const uint16_t*)(vs + (vo + 2 * (i * kD + 16 * fb))));
        }
        acc[fb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, ph, acc[fb], 0, 0, 0);
        acc[fb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, pl, acc[fb], 0, 0, 0);
      }
      // Every rank block is worked, also past m (their sums are never written): a
      // branch on m here would make the reads after it wait for every request.  Those
      // reads stay inside the tile's U_V area (30 m + 64 MK - 2 < 1024 MK bytes).
      const int uo = uwave + 2 * (4 * grp * m + c16);
#pragma unroll
      for (int ub = 0; ub < MU; ++ub) {
        bf16x4_t A;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          A[i] = __builtin_bit_cast(__bf16, *(const uint16_t*)(us + (uo + 2 * (i * m + 16 * ub))));
        uacc[ub] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, ph, uacc[ub], 0, 0, 0);
        uacc[ub] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, pl, uacc[ub], 0, 0, 0);
      }
    };
    // The tile's LDS reads are done before a later request overwrites the tile.
    auto lds_reads_done = [&]() { __builtin_amdgcn_s_waitcnt(0xc07f); };  // lgkmcnt(0)

    // The wave's tiles, two per loop pass (registers ra / rb alternate; LDS tile 0 / 1
    // with DB).
    int ti = HM ? 0 : wave;
    if (ti < ntiles) {
      KRows<MKX, Q> ra, rb;
      Pages pg_n = lookup(ti + TSTEP);
      RowAt ra_at = row_at(ti, lookup(ti)), rb_at{kOob, kOob};
      issue_k(ti, ra_at, ra);
      issue_v(ti, ra_at, Buf0{});
      while (true) {
        // tile ti: ra, LDS tile 0.  The next tile's requests go out whether or not it
        // exists (past the segment they read zeros): a request under a branch would
        // leave the join after it unsure which LDS tile is in flight, and the reads of
        // the current tile would then wait for every request.
        __builtin_amdgcn_sched_barrier(0);
        const Pages pg_nn = lookup(ti + 2 * TSTEP);
        const bool more = ti + TSTEP < ntiles;
        rb_at = row_at(ti + TSTEP, pg_n);
        issue_k(ti + TSTEP, rb_at, rb);
        if constexpr (DB) issue_v(ti + TSTEP, rb_at, Buf1{});
        __builtin_amdgcn_sched_barrier(0);
        work(ra_at, ra, Buf0{});
        if (!more) break;
        if (!DB) {
          lds_reads_done();
          issue_v(ti + TSTEP, rb_at, Buf0{});
        }
        ti += TSTEP;
        __builtin_amdgcn_sched_barrier(0);
        // tile ti: rb, LDS tile 1 (DB) or 0
        const Pages pg_n3 = lookup(ti + 2 * TSTEP);
        const bool more2 = ti + TSTEP < ntiles;
        ra_at = row_at(ti + TSTEP, pg_nn);
        issue_k(ti + TSTEP, ra_at, ra);
        if constexpr (DB) issue_v(ti + TSTEP, ra_at, Buf0{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (DB) work(rb_at, rb, Buf1{});
        else work(rb_at, rb, Buf0{});
        if (!more2) break;
        if (!DB) {
          lds_reads_done();
          issue_v(ti + TSTEP, ra_at, Buf0{});
        }
        ti += TSTEP;
        pg_n = pg_n3;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // The four lane groups of a column hold disjoint tokens' sums.
    lrun += __shfl_xor(lrun, 16);
    lrun += __shfl_xor(lrun, 32);

    // Lane (c16, grp) holds features 16 fb + 4 grp + i of the value sums and 16 ub +
    // 4 grp + i of the U_V sums of query head c16.  HM: the wave writes its head's slot.
    if constexpr (HM) {
      // value sums times V's scale, plus V_V times the U_V sums (hi and lo bf16 parts of
      // the fp32 sums, so the products keep fp32 accuracy); ranks past m count zero.
#pragma unroll
      for (int fb = 0; fb < 8; ++fb) acc[fb] *= vscale;
      if constexpr (MK > 0) {
#pragma unroll
        for (int ub = 0; ub < MU; ++ub) {
          if (16 * ub >= m) break;  // uniform
          const bool kok = 16 * ub + 4 * grp < m;
          bf16x4_t uh, ul;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = kok ? uacc[ub][i] : 0.f;
            uh[i] = (__bf16)x;
            ul[i] = (__bf16)(x - (float)uh[i]);
          }
#pragma unroll
          for (int fb = 0; fb < 8; ++fb) {
            u32x2_t w;
            if (kVVPre && ub == 0) w = vvr[kVVPre ? fb : 0];
            else w = vv_load(fb, ub);
            const bf16x4_t A = __builtin_bit_cast(bf16x4_t, w);
            acc[fb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, uh, acc[fb], 0, 0, 0);
            acc[fb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, ul, acc[fb], 0, 0, 0);
          }
        }
      }
      if (hv) {
        float* sl = wsp + (((int64_t)l * Hq + g * gq + c16) * a.slots + (s + j)) * a.slot_floats;
        if (grp == 0) {
          sl[0] = mrun;
          sl[1] = lrun;
          sl[2] = __int_as_float(j);
        }
#pragma unroll
        for (int fb = 0; fb < 8; ++fb)
          *(f32x4_t*)(sl + kAttendSlotHead + 16 * fb + 4 * grp) = acc[fb];
      }
      t0 = s1;
      continue;
    }
    // Otherwise merge the four waves' partials through LDS, then write the segment's slot.
    __syncthreads();  // every wave's tile reads are done: the tiles' LDS holds the merge
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
      float* sl = wsp + (((int64_t)l * Hq + g * gq + h) * a.slots + (s + j)) * a.slot_floats;
      if (e == 0) {
        sl[0] = M;
        sl[1] = L;
        sl[2] = __int_as_float(j);
      }
      sl[kAttendSlotHead + e] = e < kD ? A * vscale : A;
    }
    __syncthreads();  // the next segment reuses the LDS for tiles and operands
    t0 = s1;
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
  // With one wave per KV head the tile kernel has applied V_V already: the slots' value
  // sums are complete and their U_V sums unused.
  const int mv = a.heads_mapping ? 0 : m;
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
        if (d < mv) uv[u] = sl[kAttendSlotHead + kD + d];
      }
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      if (!(ls[u] > 0.f)) continue;  // the same for every thread
      if (mv > 0 && js[u] != jcur) {
        if (jcur >= 0) flush();
        jcur = js[u];
      }
      const float f = exp2f(ms[u] - M);
      den = fmaf(f, ls[u], den);
      num = fmaf(f, av[u], num);
      uk = fmaf(f, uv[u], uk);
    }
  }
  if (mv > 0 && jcur >= 0) flush();
  const int64_t o = (int64_t)l * Hq + hq;
  a.out[o * kD + d] = den > 0.f ? num / den : 0.f;
  if (a.lse != nullptr && d == 0)
    a.lse[o] = den > 0.f ? (M + log2f(den)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.splits > 0) {  // no tokens: only the merge runs, writing 0 and -inf
    const dim3 grid0((unsigned)((int64_t)a.num_layers * a.num_chunks * a.heads));
    hipLaunchKernelGGL(attend_prep, grid0, dim3(kThreads), (size_t)kD * a.rank * 2, s, a);
    // A 4-wave workgroup per (layer, split, KV head), or (HM) one wave per KV head in a
    // workgroup per (layer, split).
    const bool hm = a.heads_mapping != 0;
    const dim3 grid1((unsigned)((int64_t)a.num_layers * a.splits * (hm ? 1 : a.heads)));
    const dim3 block1((unsigned)(hm ? 64 * a.heads : kThreads));
    const int mk = (a.rank + 31) / 32;
    const bool db = a.double_buffer != 0 && mk <= 2;
#define KAMERA_ATT4(MK, PG, Q, HM)                                                             \
  do {                                                                                         \
    if (db) hipLaunchKernelGGL((attend_tiles<MK, PG, true, Q, HM>), grid1, block1, 0, s, a);   \
    else hipLaunchKernelGGL((attend_tiles<MK, PG, false, Q, HM>), grid1, block1, 0, s, a);     \
  } while (0)
#define KAMERA_ATT3(MK, PG, Q)                  \
  do {                                          \
    if (hm) KAMERA_ATT4(MK, PG, Q, true);       \
    else KAMERA_ATT4(MK, PG, Q, false);         \
  } while (0)
#define KAMERA_ATT2(MK, PG)                    \
  do {                                         \
    if (a.fp8) KAMERA_ATT3(MK, PG, true);      \
    else KAMERA_ATT3(MK, PG, false);           \
  } while (0)
#define KAMERA_ATT(MK)                              \
  do {                                              \
    if (a.page_size >= 16) KAMERA_ATT2(MK, 1);      \
    else if (a.page_size > 0) KAMERA_ATT2(MK, 2);   \
    else KAMERA_ATT2(MK, 0);                        \
  } while (0)
    if (mk == 0) KAMERA_ATT(0);
    else if (mk == 1) KAMERA_ATT(1);
    else if (mk == 2) KAMERA_ATT(2);
    else KAMERA_ATT(4);
#undef KAMERA_ATT
#undef KAMERA_ATT2
#undef KAMERA_ATT3
#undef KAMERA_ATT4
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid2((unsigned)((int64_t)a.num_layers * a.num_q_heads));
  hipLaunchKernelGGL(attend_merge, grid2, dim3(kD), 0, s, a);
  return hipGetLastError();
}

}  // namespace kamera
