// gfx950 kernels of patch formation: the top-m factors of the reuse deficit.
//
// "Kamera: KV Cache Multimodal Unificado e Invariante a Posicao para Reuso sem
// Treinamento" (gist.science/pt/paper/2606.23581), §2, "Aplicacao de Patch": the patch
// is formed once, from one conditioned forward pass and an SVD that keeps the top-m
// factors.  The forward pass is the caller's; this file takes the deficit
// Delta = KV(B|A) - KV(B|empty) of every (layer, chunk) of a channel, [T_j, F] in bf16,
// and writes U_m = U diag(s) [T_j, m] and V_m [F, m] (bf16, the layouts the reuse
// operator reads) and the singular values s (fp32).
//
// Method, per problem (layer, chunk):
//   1. G = Delta^T Delta (F x F, fp32) on MFMA 16x16x32 bf16: a dense contraction over
//      the chunk's tokens, upper-triangular 128 x 128 tiles (64 x 64 when F is not a
//      multiple of 128), mirrored.
//   2. Subspace iteration on G with k = m + 16 columns (at most 128, at most F):
//      Q <- orth(G Q) from a fixed pseudo-random start, `iters` times (fp32 tiled GEMM;
//      orth = Cholesky QR twice, Gram and Cholesky in fp64).
//   3. Rayleigh-Ritz: B = Q^T G Q (k x k), eigenpairs of B by cyclic Jacobi in LDS,
//      sorted; V_m = Q E[:, :m], s_i = sqrt(lambda_i).
//   4. U_m = Delta V_m (= U_m diag(s) of the SVD) on MFMA 16x16x32 bf16, V_m split
//      into high and low bf16 parts once per problem; rounded to bf16 with V_m.
// The top-m right singular vectors of Delta are the top-m eigenvectors of G; the error
// of the subspace iteration shrinks like (lambda_{k+1} / lambda_i)^iters.
#include <hip/hip_runtime.h>


#include "kamera_internal.h"

namespace kamera {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kThreads = 256;
constexpr int kMaxK = 128;

// A raw buffer resource over [base, base + bytes): loads at offsets past the end return
// zeros.  `opaque` keeps an offset in a vector register as computed.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ uint16_t f2bf16(float y) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(y));  // round to nearest even
}

// Workspace of one problem (floats): G [F][F], Q [F][k], Z [F][k], B [k][k], E [k][k],
// lambda [k].
struct WsLayout {
  int64_t G, Q, Z, B, E, lam, stride;
};

__host__ __device__ inline WsLayout ws_layout(int F, int k) {
  WsLayout w;
  w.G = 0;
  w.Q = w.G + (int64_t)F * F;
  w.Z = w.Q + (int64_t)F * k;
  w.B = w.Z + (int64_t)F * k;
  w.E = w.B + (int64_t)k * k;
  w.lam = w.E + (int64_t)k * k;
  w.stride = (w.lam + k + 63) / 64 * 64;
  return w;
}

// ------------------------------------------------------------------ 1. Gram on MFMA

// Workgroups go to the 8 XCDs round-robin in launch order, and each XCD has its own
// L2.  The tiles of one problem read the same data (columns of Delta, or the problem's
// workspace matrices), so the linear block index L (x fastest, then y, then z) is
// remapped to v such that each XCD takes a contiguous range of v, a bijection of
// [0, N) for N blocks: XCD x = L % 8 takes its (L / 8)-th block from the range of x.
// The kernels read their tile and problem from v in place of blockIdx.
struct Blk {
  uint32_t x, y, z;
};
__device__ __forceinline__ Blk xcd_block() {
  const uint32_t gx = gridDim.x, gxy = gx * gridDim.y, N = gxy * gridDim.z;
  const uint32_t L = blockIdx.x + blockIdx.y * gx + blockIdx.z * gxy;
  const uint32_t x = L & 7u, s = L >> 3, Q = N >> 3, R = N & 7u;
  uint32_t v = (x < R ? x * (Q + 1) : R * (Q + 1) + (x - R) * Q) + s;
  Blk r;
  r.z = v / gxy;
  v -= r.z * gxy;
  r.y = v / gx;
  r.x = v - r.y * gx;
  return r;
}

// One 64 x 64 tile (ti <= tj) of G = Delta_j^T Delta_j.  Per 32-token step the
// workgroup stages both 64-feature column blocks of Delta transposed in LDS
// ([feature][token]), so each lane reads the 8 consecutive tokens of one feature that
// an MFMA operand row holds.  Wave w owns the 32 x 32 quadrant (w >> 1, w & 1): 2 x 2
// MFMA 16x16x32 tiles.  G[i][j] = sum_t A[i][t] B[t][j] with A = Delta^T, B = Delta.
__global__ __launch_bounds__(kThreads) void gram_tiles(FormArgs P, int64_t p0, float* Gbase,
                                                       int64_t gstride) {
  const int ntile = P.F / 64;
  const Blk bk = xcd_block();
  const int prob = (int)bk.y;
  int rem = (int)bk.x, ti = 0;
  while (rem >= ntile - ti) {
    rem -= ntile - ti;
    ++ti;
  }
  const int tj = ti + rem;
  const int64_t p = p0 + prob;
  const int64_t layer = p / P.num_chunks;
  const int j = (int)(p - layer * P.num_chunks);
  // Rows [a, b) of the chunk, kept inside [0, total_tokens) whatever the offsets hold.
  const int64_t a = min(max(P.offsets[j], (int64_t)0), P.total_tokens);
  const int64_t b = min(max(P.offsets[j + 1], a), P.total_tokens);
  float* G = Gbase + (int64_t)prob * gstride;

  __shared__ __attribute__((aligned(16))) uint16_t sA[64][40];  // 32 tokens + 8 pad
  __shared__ __attribute__((aligned(16))) uint16_t sB[64][40];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int tl = tid >> 3, c8 = (tid & 7) * 8;
  const uint16_t* D = P.delta + layer * P.total_tokens * P.F;
  f32x4_t acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t t0 = a; t0 < b; t0 += 32) {
    const int64_t tt = t0 + tl;
    u32x4_t va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
    if (tt < b) {
      va = *(const u32x4_t*)(D + tt * P.F + ti * 64 + c8);
      vb = *(const u32x4_t*)(D + tt * P.F + tj * 64 + c8);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sA[c8 + 2 * e][tl] = (uint16_t)(va[e] & 0xffffu);
      sA[c8 + 2 * e + 1][tl] = (uint16_t)(va[e] >> 16);
      sB[c8 + 2 * e][tl] = (uint16_t)(vb[e] & 0xffffu);
      sB[c8 + 2 * e + 1][tl] = (uint16_t)(vb[e] >> 16);
    }
    __syncthreads();
    const int g = lane >> 4, r16 = lane & 15;
    bf16x8_t fa[2], fb[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      fa[x] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)&sA[wi * 32 + x * 16 + r16][8 * g]);
      fb[x] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)&sB[wj * 32 + x * 16 + r16][8 * g]);
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
        acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[x], fb[y], acc[x][y], 0, 0, 0);
    __syncthreads();
  }
  // D layout: lane holds rows 4g .. 4g + 3 of column lane & 15.
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gi = ti * 64 + wi * 32 + x * 16 + 4 * g + r;
        const int gj = tj * 64 + wj * 32 + y * 16 + c;
        G[(int64_t)gi * P.F + gj] = acc[x][y][r];
        if (ti != tj) G[(int64_t)gj * P.F + gi] = acc[x][y][r];
      }
}

// The same for widths that are multiples of 128, with 128 x 128 tiles: wave w owns the
// 64 x 64 quadrant (w >> 1, w & 1), 4 x 4 MFMA tiles, so each 64-token step issues 32
// MFMAs per wave between barriers.  The next step's rows are loaded into registers
// before the current step's MFMAs; rows go to LDS transposed two tokens at a time
// (one 32-bit word holds a feature's pair of tokens).
// Used where a chunk's rows span 2^31 - 64 bytes or more (the buffer resources of
// gram_tr cannot reach them).
__global__ __launch_bounds__(kThreads) void gram_tiles128(FormArgs P, int64_t p0, float* Gbase,
                                                          int64_t gstride) {
  const int ntile = P.F / 128;
  const Blk bk = xcd_block();
  const int prob = (int)bk.y;
  int rem = (int)bk.x, ti = 0;
  while (rem >= ntile - ti) {
    rem -= ntile - ti;
    ++ti;
  }
  const int tj = ti + rem;
  const int64_t p = p0 + prob;
  const int64_t layer = p / P.num_chunks;
  const int j = (int)(p - layer * P.num_chunks);
  const int64_t a = min(max(P.offsets[j], (int64_t)0), P.total_tokens);
  const int64_t b = min(max(P.offsets[j + 1], a), P.total_tokens);
  float* G = Gbase + (int64_t)prob * gstride;

  constexpr int KS = 64;           // tokens per LDS step
  constexpr int RS = KS / 2 + 4;   // 32-bit words per LDS row (token pairs + pad)
  __shared__ __attribute__((aligned(16))) uint32_t sA[128][RS];
  __shared__ __attribute__((aligned(16))) uint32_t sB[128][RS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const uint16_t* D = P.delta + layer * P.total_tokens * P.F;
  // Thread tid reads feature group fg = tid & 15 (8 features) of the 4 tokens
  // 4 tq .. 4 tq + 3, tq = tid >> 4: 16 consecutive lanes read 256 contiguous bytes of
  // one row, and a wave instruction touches 4 rows.  In LDS, the word of token pair tp
  // of feature f sits at column tp ^ 4 ((f >> 4) & 7): the swizzle moves whole 16-byte
  // groups, so an MFMA operand (4 words of one feature) stays one aligned 16-byte read,
  // and a thread's two words per feature (token pairs 2 tq, 2 tq + 1) stay one aligned
  // 8-byte store; a wave's stores spread evenly over the 64 banks.
  const int fg = tid & 15, tq = tid >> 4;
  const int col = (2 * tq) ^ (4 * ((fg >> 1) & 7));  // (f >> 4) & 7 for every f of the group
  auto load = [&](int64_t t0, int col0, u32x4_t (&r)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t t = t0 + 4 * tq + u;
      r[u] = u32x4_t{0u, 0u, 0u, 0u};
      if (t < b) r[u] = *(const u32x4_t*)(D + t * P.F + col0 + fg * 8);
    }
  };
  auto store = [&](uint32_t (*S)[RS], const u32x4_t (&r)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // features 2e, 2e + 1 of the group
      u32x2_t lo, hi;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const uint32_t w0 = r[2 * pp][e], w1 = r[2 * pp + 1][e];
        lo[pp] = (w0 & 0xffffu) | (w1 << 16);
        hi[pp] = (w0 >> 16) | (w1 & 0xffff0000u);
      }
      *(u32x2_t*)&S[fg * 8 + 2 * e][col] = lo;
      *(u32x2_t*)&S[fg * 8 + 2 * e + 1][col] = hi;
    }
  };
  f32x4_t acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t ra[4], rb[4];
  if (a < b) {
    load(a, ti * 128, ra);
    load(a, tj * 128, rb);
  }
  const int g = lane >> 4, r16 = lane & 15;
  for (int64_t t0 = a; t0 < b; t0 += KS) {
    __syncthreads();  // the previous step's fragments are read
    store(sA, ra);
    store(sB, rb);
    __syncthreads();
    if (t0 + KS < b) {
      load(t0 + KS, ti * 128, ra);
      load(t0 + KS, tj * 128, rb);
    }
#pragma unroll
    for (int ks = 0; ks < KS / 32; ++ks) {
      bf16x8_t fa[4], fb[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {  // rows wi * 64 + x * 16 + r16: (row >> 4) & 7 = wi * 4 + x
        const int ca = (ks * 16 + 4 * g) ^ (4 * (wi * 4 + x));
        const int cb = (ks * 16 + 4 * g) ^ (4 * (wj * 4 + x));
        fa[x] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)&sA[wi * 64 + x * 16 + r16][ca]);
        fb[x] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)&sB[wj * 64 + x * 16 + r16][cb]);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
  }
  const int c = lane & 15;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gi = ti * 128 + wi * 64 + x * 16 + 4 * g + r;
        const int gj = tj * 128 + wj * 64 + y * 16 + c;
        G[(int64_t)gi * P.F + gj] = acc[x][y][r];
        if (ti != tj) G[(int64_t)gj * P.F + gi] = acc[x][y][r];
      }
}

// The same 128 x 128 tiles with the rows staged in LDS as they lie in memory.  Each
// 64-token step's rows of both 128-feature column blocks go straight from memory into
// one of two LDS stages (16 bytes per lane per request, no registers held), one step
// ahead of the MFMAs; deeper rings measured slower (each wave's requests run further
// ahead of the other tiles of its problem, whose reads of the same rows then miss the
// L2 more often).  The MFMA operands come from the untransposed rows through the
// gfx950 transposing LDS read: within each 16-lane group, lane i receives as its
// element e element i & 3 of the 8 bytes that lane 4 e + (i >> 2) addressed.  So when
// lane s of group g addresses row 8 g + 4 h + (s >> 2) at features f + 4 (s & 3),
// lane i holds feature f + i of rows 8 g + 4 h .. 8 g + 4 h + 3: half of its MFMA
// operand (the tokens are the contraction index).  A row is 256 bytes, all 64 banks;
// its 32-byte slot q sits at slot q ^ sw(r), sw(r) = (r & 3) | ((r >> 3) & 1) << 2, so
// the eight rows a half-wave reads fall in eight different slots.  One barrier per
// step: the stage a step's requests overwrite was read in the step before.
constexpr uint32_t kGramOob = 0x80000000u;  // past every chunk: such requests read zeros

__device__ __forceinline__ void lds_dma16(rsrc_t r, uint32_t off, unsigned char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           (int)opaque(off), 0, 0, 0);
}
// Waits until at most n vector-memory requests of this wave are outstanding.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2_t lds_tr16(const unsigned char* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (__attribute__((address_space(3))) i16x4_t*)p));
}

__global__ __launch_bounds__(kThreads) void gram_tr(FormArgs P, int64_t p0, float* Gbase,
                                                    int64_t gstride) {
  constexpr int KS = 64;                  // tokens per step
  constexpr int kStage = KS * 256;        // bytes of one block's rows in one step
  constexpr int kSeg = kStage / 4096;     // 1 KB requests per wave, per block and step
  const int ntile = P.F / 128;
  const Blk bk = xcd_block();
  const int prob = (int)bk.y;
  int rem = (int)bk.x, ti = 0;
  while (rem >= ntile - ti) {
    rem -= ntile - ti;
    ++ti;
  }
  const int tj = ti + rem;
  const int64_t p = p0 + prob;
  const int64_t layer = p / P.num_chunks;
  const int j = (int)(p - layer * P.num_chunks);
  const int64_t a = min(max(P.offsets[j], (int64_t)0), P.total_tokens);
  const int64_t b = min(max(P.offsets[j + 1], a), P.total_tokens);
  float* G = Gbase + (int64_t)prob * gstride;
  const uint16_t* D = P.delta + layer * P.total_tokens * P.F;
  const int64_t nrows = b - a;
  const rsrc_t rd = make_rsrc(D + a * P.F, (uint32_t)(nrows * P.F * 2));

  // Stage k: block ti's rows at bytes [0, kStage), block tj's at [kStage, 2 kStage).  A
  // diagonal tile (ti == tj) reads both operands from the first half; its requests for
  // the second go past the chunk (no memory traffic, zeros) to keep the count uniform.
  // One array per stage: the compiler then waits for exactly the requests a read needs.
  __shared__ __attribute__((aligned(1024))) unsigned char st0[2 * kStage], st1[2 * kStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave >> 1, wj = wave & 1;
  const bool diag = ti == tj;

  // Requests: this wave's segment jj = wave * kSeg + i of a block (bytes 1024 jj ..)
  // holds rows 4 jj .. 4 jj + 3; lane l writes 16-byte group l & 15 of row
  // 4 jj + (l >> 4), which holds the row's logical group (l & 15) ^ 2 sw(row).
  const int rq = lane >> 4, gp = lane & 15;
  uint32_t colA[kSeg], colB[kSeg];
#pragma unroll
  for (int i = 0; i < kSeg; ++i) {
    const int jj = wave * kSeg + i;
    const int sw = rq | (((jj >> 1) & 1) << 2);
    const int lg = gp ^ (2 * sw);
    colA[i] = 2u * (uint32_t)(ti * 128 + 8 * lg);
    colB[i] = 2u * (uint32_t)(tj * 128 + 8 * lg);
  }
  auto issue = [&](unsigned char* dst, int64_t st) {
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      const int jj = wave * kSeg + i;
      const int64_t row = st * KS + 4 * jj + rq;
      const uint32_t ro = row < nrows ? (uint32_t)(row * P.F * 2) : kGramOob;
      lds_dma16(rd, ro + colA[i], dst + 1024 * jj);
      lds_dma16(rd, diag ? kGramOob : ro + colB[i], dst + kStage + 1024 * jj);
    }
  };
  // Operand reads: lane (s, g), s = lane & 15, g = lane >> 4.  Row 32 ks + 8 g + 4 h +
  // (s >> 2) has sw = (s >> 2) | (g & 1) << 2 whatever ks and h are.
  const int s16 = lane & 15, g = lane >> 4;
  const int swr = (s16 >> 2) | ((g & 1) << 2);
  const int rbase = (8 * g + (s16 >> 2)) * 256 + 8 * (s16 & 3);
  const int bhalf = diag ? 0 : kStage;
  int offA[4], offB[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    offA[x] = rbase + 32 * ((wi * 4 + x) ^ swr);
    offB[x] = bhalf + rbase + 32 * ((wj * 4 + x) ^ swr);
  }
  f32x4_t acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const unsigned char* src) {
#pragma unroll
    for (int ks = 0; ks < KS / 32; ++ks) {
      bf16x8_t fa[4], fb[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const u32x2_t a0 = lds_tr16(src + ks * 32 * 256 + offA[x]);
        const u32x2_t a1 = lds_tr16(src + ks * 32 * 256 + 4 * 256 + offA[x]);
        const u32x2_t b0 = lds_tr16(src + ks * 32 * 256 + offB[x]);
        const u32x2_t b1 = lds_tr16(src + ks * 32 * 256 + 4 * 256 + offB[x]);
        fa[x] = __builtin_bit_cast(bf16x8_t, u32x4_t{a0[0], a0[1], a1[0], a1[1]});
        fb[x] = __builtin_bit_cast(bf16x8_t, u32x4_t{b0[0], b0[1], b1[0], b1[1]});
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
  };
  // Step st reads stage st % 2.  Before it, this wave's requests of that stage are done
  // (vmcnt 0: the other stage's were issued after the previous step's reads); the
  // barrier makes every wave's done, and every wave has read the other stage, which the
  // next step's requests then refill.
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  const int64_t nsteps = (nrows + KS - 1) / KS;
  issue(st0, 0);
  int64_t st = 0;
  while (st < nsteps) {
    wait_vm<0>();
    barrier();
    issue(st1, st + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(st0);
    if (++st >= nsteps) break;
    wait_vm<0>();
    barrier();
    issue(st0, st + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(st1);
    ++st;
  }
  // Requests past the last step (zeros) are still in flight: done before the wave ends.
  wait_vm<0>();
  const int c = lane & 15;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gi = ti * 128 + wi * 64 + x * 16 + 4 * g + r;
        const int gj = tj * 128 + wj * 64 + y * 16 + c;
        G[(int64_t)gi * P.F + gj] = acc[x][y][r];
        if (ti != tj) G[(int64_t)gj * P.F + gi] = acc[x][y][r];
      }
}

// ------------------------------------------------------------------ 2. dense fp32 algebra

// Fixed pseudo-random start: entry e of Q (row-major F x k) is a 32-bit integer hash of
// e (a multiply-xorshift mixer) scaled to [-1, 1); the same for every problem.
__global__ __launch_bounds__(kThreads) void init_start(FormArgs P) {
  const WsLayout W = ws_layout(P.F, P.k);
  float* Q = P.ws + (int64_t)blockIdx.y * W.stride + W.Q;
  const int n = P.F * P.k;
  for (int e = blockIdx.x * kThreads + threadIdx.x; e < n; e += gridDim.x * kThreads) {
    uint32_t h = (uint32_t)e * 0x9E3779B9u + 0x7F4A7C15u;
    h ^= h >> 16;
    h *= 0x7feb352du;
    h ^= h >> 15;
    h *= 0x846ca68bu;
    h ^= h >> 16;
    Q[e] = (float)(int32_t)h * 0x1p-31f;
  }
}

// C = op(A) B for every problem of the batch (grid z): op(A) is M x K (A row-major
// M x K, or with TA row-major K x M), B row-major K x N, C row-major M x N, fp32.  Every
// call has N = k <= 128, so one tile spans all columns, 16 NT of them with NT = N / 16
// rounded up, on fp32 MFMA (below).  Two forms:
//   - TM = 64 rows, 16-deep LDS steps, wave w the rows 16 w .. + 15 over all of K;
//   - SPLIT: TM = 16 rows, 64-deep LDS steps, wave w the 16-deep slice w of each step
//     (K split over the waves), the four partial tiles summed through LDS at the end.
//     It runs 4x the workgroups and a quarter of the serial steps, for launches whose
//     64-row grid cannot fill the chip; it re-reads B per 16 rows instead of per 64.
// Offsets are element offsets inside each problem's workspace.
template <bool TA, int NT, bool SPLIT>
__global__ __launch_bounds__(kThreads) void gemm_ws(FormArgs P, int64_t a_off, int lda,
                                                     int64_t b_off, int ldb, int64_t c_off,
                                                     int ldc, int M, int N, int K) {
  constexpr int TN = 16 * NT;
  constexpr int TM = SPLIT ? 16 : 64;
  constexpr int KS = SPLIT ? 64 : 16;  // K per LDS step
  const WsLayout W = ws_layout(P.F, P.k);
  const Blk bk = xcd_block();
  float* base = P.ws + (int64_t)bk.z * W.stride;
  const float* A = base + a_off;
  const float* B = base + b_off;
  float* C = base + c_off;
  __shared__ float sA[KS][TM + (SPLIT ? 1 : 4)];  // [k][row]
  __shared__ __attribute__((aligned(16))) float sB[KS][TN + 4];
  const int tid = threadIdx.x;
  const int m0 = (int)bk.y * TM;
  // fp32 MFMA (v_mfma_f32_16x16x4_f32): lane l feeds A[row l & 15][k l >> 4] and
  // B[k l >> 4][col l & 15] and holds C[4 (l >> 4) + q][l & 15], q < 4, of each of the
  // NT 16 x 16 tiles.
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lk = lane >> 4;
  const int wrow = SPLIT ? 0 : 16 * wave;  // the wave's rows in the tile
  const int wk = SPLIT ? 16 * wave : 0;    // and its k slice in a step
  f32x4_t acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += KS) {
#pragma unroll
    for (int q = 0; q < TM * KS / kThreads; ++q) {  // A: TM x KS
      const int idx = tid + kThreads * q;
      int r, kk;
      if (TA) {
        kk = idx / TM;
        r = idx % TM;
      } else {
        r = idx / KS;
        kk = idx % KS;
      }
      const int gm = m0 + r, gk = k0 + kk;
      float v = 0.f;
      if (gm < M && gk < K) v = TA ? A[(int64_t)gk * lda + gm] : A[(int64_t)gm * lda + gk];
      sA[kk][r] = v;
    }
#pragma unroll
    for (int q = 0; q < KS * TN / kThreads; ++q) {  // B: KS x TN
      const int idx = tid + kThreads * q;
      const int bkk = idx / TN, bc = idx % TN;
      const int gbk = k0 + bkk;
      sB[bkk][bc] = (gbk < K && bc < N) ? B[(int64_t)gbk * ldb + bc] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = wk; kk < wk + 16; kk += 4) {
      const float av = sA[kk + lk][wrow + l16];
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, sB[kk + lk][16 * j + l16], acc[j], 0,
                                                      0, 0);
    }
    __syncthreads();
  }
  if constexpr (SPLIT) {
    // Waves 1..3 leave their partial tiles in sB's memory (3 NT x 64 x 16 bytes, within
    // sB's 64 x (16 NT + 4) floats); wave 0 adds them.
    f32x4_t* red = reinterpret_cast<f32x4_t*>(&sB[0][0]);
    if (wave > 0) {
#pragma unroll
      for (int j = 0; j < NT; ++j) red[((wave - 1) * NT + j) * 64 + lane] = acc[j];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int w = 0; w < 3; ++w) acc[j] += red[(w * NT + j) * 64 + lane];
  }
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int gm = m0 + wrow + 4 * lk + q, gn = 16 * j + l16;
      if (gm < M && gn < N) C[(int64_t)gm * ldc + gn] = acc[j][q];
    }
}

// Launch of gemm_ws for `count` problems, N <= 128: the K-split form when the 64-row
// grid would leave CUs idle (fewer than 256 workgroups).  Measured on G Q products:
// 224 workgroups (width 512, 28 problems) 55 -> 38 us with the split; 256 (width 1024,
// 16 problems) slower with it; 1024 (width 1024, 64 problems) 254 -> 706 us.
template <bool TA>
void launch_gemm_ws(const FormArgs& P, int count, hipStream_t s, int64_t a_off, int lda,
                    int64_t b_off, int ldb, int64_t c_off, int ldc, int M, int N, int K) {
  const bool split = (int64_t)((M + 63) / 64) * count < 256;
  const dim3 g(1, split ? (M + 15) / 16 : (M + 63) / 64, count), blk(kThreads);
#define KAMERA_GEMM_WS(NT)                                                                    \
  case NT:                                                                                    \
    if (split)                                                                                \
      hipLaunchKernelGGL((gemm_ws<TA, NT, true>), g, blk, 0, s, P, a_off, lda, b_off, ldb,    \
                         c_off, ldc, M, N, K);                                                \
    else                                                                                      \
      hipLaunchKernelGGL((gemm_ws<TA, NT, false>), g, blk, 0, s, P, a_off, lda, b_off, ldb,   \
                         c_off, ldc, M, N, K);                                                \
    break
  switch ((N + 15) / 16) {
    KAMERA_GEMM_WS(1);
    KAMERA_GEMM_WS(2);
    KAMERA_GEMM_WS(3);
    KAMERA_GEMM_WS(4);
    KAMERA_GEMM_WS(5);
    KAMERA_GEMM_WS(6);
    KAMERA_GEMM_WS(7);
    KAMERA_GEMM_WS(8);
    default: break;  // N <= k <= 128 (kMaxK)
  }
#undef KAMERA_GEMM_WS
}

// Block reduction of one float over the workgroup (result in every thread).
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// W = X^T X in fp64 for the F x k matrix X (Z or Q) of every problem: one 32 x 32 tile
// of W per workgroup.  The F rows are split over the four waves (F is a multiple of 64):
// wave w stages rows w F / 4 + 16 s .. + 15 of step s in its own LDS slice and
// accumulates the whole tile over its quarter, 4 x 4 outputs per lane, so each wave
// walks F / 64 steps; the four partial tiles are summed through LDS.  W occupies the B
// and E regions of the workspace (2 k^2 floats = k^2 doubles).
__global__ __launch_bounds__(kThreads) void gram64(FormArgs P, int64_t x_off) {
  const WsLayout W = ws_layout(P.F, P.k);
  const Blk bk = xcd_block();
  float* base = P.ws + (int64_t)bk.z * W.stride;
  const float* X = base + x_off;
  double* Wd = reinterpret_cast<double*>(base + W.B);
  const int k = P.k, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ty = lane >> 3, tx = lane & 7;  // outputs 4 ty + a, 4 tx + b
  const int i0 = (int)bk.y * 32, j0 = (int)bk.x * 32;
  const int quarter = P.F / 4, fw = wave * quarter;
  __shared__ float si[4][16][33], sj[4][16][33];
  __shared__ double red[3][16][64];
  double acc[4][4] = {};
  for (int f0 = 0; f0 < quarter; f0 += 16) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {  // the wave's 16 x 32 slices of both column blocks
      const int idx = lane + 64 * q;
      const int r = idx >> 5, c = idx & 31;
      const int64_t row = (int64_t)(fw + f0 + r) * k;
      si[wave][r][c] = (i0 + c < k) ? X[row + i0 + c] : 0.f;
      sj[wave][r][c] = (j0 + c < k) ? X[row + j0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      double xi[4], xj[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        xi[a] = (double)si[wave][r][4 * ty + a];
        xj[a] = (double)sj[wave][r][4 * tx + a];
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(xi[a], xj[b], acc[a][b]);
    }
    __syncthreads();
  }
  if (wave > 0) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) red[wave - 1][4 * a + b][lane] = acc[a][b];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const double v = acc[a][b] + red[0][4 * a + b][lane] + red[1][4 * a + b][lane] +
                       red[2][4 * a + b][lane];
      const int i = i0 + 4 * ty + a, jj = j0 + 4 * tx + b;
      if (i < k && jj < k) Wd[(int64_t)i * k + jj] = v;
    }
}

// R^-1 of the Cholesky QR of one problem: W = X^T X (fp64, from gram64) is factored
// W = L L^T column by column in LDS, in fp64; a column whose pivot falls below 1e-12 of
// its diagonal (its remainder after projection is under 1e-6 of its norm: a direction
// the chunk does not span) is dropped.  L is then inverted in place (columns from the
// last, each from the already inverted trailing block), and R^-1 = L^-T is written as
// fp32 k x k into the B region, so that X R^-1 has orthonormal (or zero) columns.
__global__ __launch_bounds__(kThreads) void chol_rinv(FormArgs P) {
  const WsLayout W = ws_layout(P.F, P.k);
  float* base = P.ws + (int64_t)blockIdx.x * W.stride;
  const double* Wd = reinterpret_cast<const double*>(base + W.B);
  float* Rinv = base + W.B;
  const int k = P.k, tid = threadIdx.x;
  __shared__ double L[kMaxK][kMaxK + 1];
  __shared__ double col[kMaxK];
  __shared__ double dg[kMaxK];  // L's diagonal, moved into L once the factor is done
  for (int e = tid; e < k * k; e += kThreads) L[e / k][e % k] = Wd[e];
  __syncthreads();
  for (int i = tid; i < k; i += kThreads) col[i] = L[i][i];  // diagonal of W
  __syncthreads();
  // Column j: every thread reads the pivot L[j][j], which no thread writes during the
  // column (the scaling writes rows below j, the update columns right of j), so one
  // barrier after the scaling and one after the update order the steps.
  for (int j = 0; j < k; ++j) {
    const double d = L[j][j];
    const bool keep = d > 1e-12 * col[j] && d > 0.0;
    const double inv = keep ? 1.0 / sqrt(d) : 0.0;
    for (int i = j + 1 + tid; i < k; i += kThreads) L[i][j] *= inv;
    if (tid == 0) dg[j] = keep ? sqrt(d) : 0.0;
    __syncthreads();
    // Trailing update L[i][c] -= L[i][j] L[c][j], j < c <= i, on a 16 x 16 thread grid
    // (rows by tid >> 4, columns by tid & 15).
    const int n = k - j - 1;
    for (int r = tid >> 4; r < n; r += 16) {
      const int ii = j + 1 + r;
      const double lij = L[ii][j];
      for (int c = tid & 15; c <= r; c += 16) L[ii][j + 1 + c] -= lij * L[j + 1 + c][j];
    }
    __syncthreads();
  }
  for (int i = tid; i < k; i += kThreads) L[i][i] = dg[i];
  __syncthreads();
  // In-place inverse of the lower-triangular L (dropped columns stay zero).  For column
  // j, row i needs -(Linv[i][j+1..i] . L[j+1..i][j]) djj: four lanes share a row, each
  // summing every fourth term, and two lane exchanges combine them.
  for (int j = k - 1; j >= 0; --j) {
    const double djj = L[j][j] > 0.0 ? 1.0 / L[j][j] : 0.0;
    const int n = k - j - 1;
    for (int r0 = 0; r0 < n; r0 += kThreads / 4) {
      const int r = r0 + (tid >> 2), q = tid & 3, i = j + 1 + r;
      double s = 0.0;
      if (r < n)
        for (int p2 = j + 1 + q; p2 <= i; p2 += 4) s += L[i][p2] * L[p2][j];
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      if (r < n && q == 0) col[i] = -s * djj;
    }
    __syncthreads();
    for (int i = j + 1 + tid; i < k; i += kThreads) L[i][j] = col[i];
    if (tid == 0) L[j][j] = djj;
    __syncthreads();
  }
  for (int e = tid; e < k * k; e += kThreads) {  // R^-1[i][j] = Linv[j][i]
    const int i = e / k, jj = e % k;
    Rinv[e] = jj >= i ? (float)L[jj][i] : 0.f;
  }
}

// ------------------------------------------------------------------ 3. Jacobi on B

// Eigenpairs of the symmetric k x k matrix B by cyclic Jacobi in LDS (round-robin
// ordering: k/2 disjoint rotations per step, k - 1 steps per sweep, sweeps until the
// off-diagonal squared mass is below 1e-10 of the total, at most 30; fp32 rounding
// keeps it near (k eps)^2 of the total, below that bound).  Writes the eigenvectors
// sorted by decreasing eigenvalue to E (k x k, column c = c-th) and the eigenvalues to
// lambda.
__global__ __launch_bounds__(kThreads) void jacobi_eig(FormArgs P) {
  const WsLayout W = ws_layout(P.F, P.k);
  float* base = P.ws + (int64_t)blockIdx.x * W.stride;
  const int k = P.k, tid = threadIdx.x;
  __shared__ float A[kMaxK][kMaxK + 1];
  __shared__ float V[kMaxK][kMaxK + 1];
  __shared__ float cs[kMaxK / 2], sn[kMaxK / 2];
  __shared__ int pp[kMaxK / 2], qq[kMaxK / 2];
  __shared__ float red[4];
  __shared__ int rank_of[kMaxK];
  for (int e = tid; e < k * k; e += kThreads) {
    const int i = e / k, j = e % k;
    // symmetrize: B = Q^T G Q is symmetric up to rounding
    A[i][j] = 0.5f * (base[W.B + (int64_t)i * k + j] + base[W.B + (int64_t)j * k + i]);
    V[i][j] = i == j ? 1.f : 0.f;
  }
  __syncthreads();
  const int half = k / 2;
  // The rotation loops take elements e = tid, tid + kThreads, ... of a half x k array as
  // (pair e / k, index e % k); both advance by fixed steps, so no loop divides.
  const int r_init = tid / k, j_init = tid - r_init * k;
  const int dq = kThreads / k, dr = kThreads - dq * k;
  for (int sweep = 0; sweep < 30; ++sweep) {
    float off = 0.f, tot = 0.f;
    for (int e = tid; e < k * k; e += kThreads) {
      const int i = e / k, j = e % k;
      const float v = A[i][j] * A[i][j];
      tot += v;
      if (i != j) off += v;
    }
    off = block_sum(off, red);
    tot = block_sum(tot, red);
    if (!(off > 1e-10f * tot) || tot == 0.f) break;
    for (int step = 0; step < k - 1; ++step) {
      // Round-robin pairs: player 0 fixed, the others rotate by `step`.
      if (tid < half) {
        int a = tid == 0 ? 0 : 1 + (tid - 1 + step) % (k - 1);
        int b = 1 + (k - 2 - tid + step) % (k - 1);
        if (a > b) {
          const int t = a;
          a = b;
          b = t;
        }
        pp[tid] = a;
        qq[tid] = b;
        const float apq = A[a][b];
        float c = 1.f, s = 0.f;
        if (apq != 0.f) {
          const float theta = (A[b][b] - A[a][a]) / (2.f * apq);
          const float t = copysignf(1.f, theta) / (fabsf(theta) + sqrtf(fmaf(theta, theta, 1.f)));
          c = rsqrtf(fmaf(t, t, 1.f));
          s = t * c;
        }
        cs[tid] = c;
        sn[tid] = s;
      }
      __syncthreads();
      // rows p, q of A
      for (int r = r_init, j = j_init; r < half;) {
        const int p = pp[r], q = qq[r];
        const float c = cs[r], s = sn[r];
        const float ap = A[p][j], aq = A[q][j];
        A[p][j] = c * ap - s * aq;
        A[q][j] = s * ap + c * aq;
        j += dr;
        r += dq;
        if (j >= k) {
          j -= k;
          ++r;
        }
      }
      __syncthreads();
      // columns p, q of A and of V
      for (int r = r_init, i = j_init; r < half;) {
        const int p = pp[r], q = qq[r];
        const float c = cs[r], s = sn[r];
        const float ap = A[i][p], aq = A[i][q];
        A[i][p] = c * ap - s * aq;
        A[i][q] = s * ap + c * aq;
        const float vp = V[i][p], vq = V[i][q];
        V[i][p] = c * vp - s * vq;
        V[i][q] = s * vp + c * vq;
        i += dr;
        r += dq;
        if (i >= k) {
          i -= k;
          ++r;
        }
      }
      __syncthreads();
    }
  }
  // Sort by decreasing eigenvalue (ties by index).
  for (int i = tid; i < k; i += kThreads) {
    const float li = A[i][i];
    int r = 0;
    for (int j = 0; j < k; ++j) {
      const float lj = A[j][j];
      r += (lj > li || (lj == li && j < i)) ? 1 : 0;
    }
    rank_of[i] = r;
  }
  __syncthreads();
  for (int e = tid; e < k * k; e += kThreads) {
    const int i = e / k, j = e % k;  // V[i][j]: component i of eigenvector j
    base[W.E + (int64_t)i * k + rank_of[j]] = V[i][j];
  }
  for (int j = tid; j < k; j += kThreads) base[W.lam + rank_of[j]] = A[j][j];
}

// ------------------------------------------------------------------ 4. outputs

// V_m (bf16, [F][m] of this layer and chunk) from the first m columns of the F x k
// array at v_off, where the caller put Q E; s = sqrt(max(lambda, 0)).
__global__ __launch_bounds__(kThreads) void write_v(FormArgs P, int64_t p0, int64_t v_off) {
  const WsLayout W = ws_layout(P.F, P.k);
  const float* base = P.ws + (int64_t)blockIdx.y * W.stride;
  const int64_t p = p0 + blockIdx.y;
  uint16_t* Vo = P.V_out + p * (int64_t)P.F * P.m;
  for (int e = blockIdx.x * kThreads + threadIdx.x; e < P.F * P.m; e += gridDim.x * kThreads) {
    const int f = e / P.m, c = e % P.m;
    Vo[e] = f2bf16(c < P.k ? base[v_off + (int64_t)f * P.k + c] : 0.f);
  }
  if (blockIdx.x == 0 && P.sigma_out != nullptr)
    for (int c = threadIdx.x; c < P.m; c += kThreads)
      P.sigma_out[p * P.m + c] = c < P.k ? sqrtf(fmaxf(base[W.lam + c], 0.f)) : 0.f;
}

// U_m = Delta V_m on MFMA (v_mfma_f32_16x16x32_bf16).  V_m (fp32, F x k at v_off) is
// split into high and low bf16 parts (x - hi - lo <= 2^-17 |x|): the bf16 x bf16
// products with Delta are exact and accumulate in fp32, so the sums match an fp32
// product to fp32 rounding.

constexpr int kUSteps = 2;  // 32-feature MFMA steps per staged 64-feature block

// The split, once per problem, into the G region of the workspace, which is free once
// the Rayleigh-Ritz products are done.  Only the first mu = min(m, k) columns of V_m can
// be nonzero; they take nv = mu / 16 rounded up column tiles, and 16 nv <= F (k <= F,
// and F is a multiple of 64), so the F * 16 nv floats fit in G's F^2.  For each
// 64-feature block: 16-byte B fragments [part][step][column tile][lane], in the order
// `write_u_mfma` stages them.  Lane (c16, g) of column tile ct, step st holds features
// 64 fb + 32 st + 8 g .. + 7 of column 16 ct + c16 (zero from column mu on).
__global__ __launch_bounds__(kThreads) void split_vm(FormArgs P, int64_t v_off) {
  const WsLayout W = ws_layout(P.F, P.k);
  const float* Vm = P.ws + (int64_t)blockIdx.y * W.stride + v_off;
  u32x4_t* out = reinterpret_cast<u32x4_t*>(P.ws + (int64_t)blockIdx.y * W.stride + W.G);
  const int k = P.k, mu = min(P.m, k), nct = (mu + 15) / 16;
  const int n = (P.F / 64) * kUSteps * nct * 64;
  for (int idx = blockIdx.x * kThreads + threadIdx.x; idx < n; idx += gridDim.x * kThreads) {
    const int l = idx & 63;
    int rest = idx >> 6;
    const int ct = rest % nct;
    rest /= nct;
    const int st = rest % kUSteps, fb = rest / kUSteps;
    const int col = 16 * ct + (l & 15);
    const int f8 = 64 * fb + 32 * st + 8 * (l >> 4);
    bf16x8_t hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = col < mu ? Vm[(int64_t)(f8 + e) * k + col] : 0.f;
      hi[e] = (__bf16)x;
      lo[e] = (__bf16)(x - (float)hi[e]);
    }
    const int64_t blk = (int64_t)fb * 2 * kUSteps * nct * 64;
    out[blk + (st * nct + ct) * 64 + l] = __builtin_bit_cast(u32x4_t, hi);
    out[blk + ((kUSteps + st) * nct + ct) * 64 + l] = __builtin_bit_cast(u32x4_t, lo);
  }
}

// The product: 64-token tiles of the chunk, tile blockIdx.x + i * gridDim.x for
// i = 0, 1, ... in workgroup x; wave w takes the 16-token slice w of a tile.  Every
// 64 features the workgroup copies that block's fragments into LDS; each lane loads its
// A fragment, 8 consecutive features of token c16 of its wave's tile, straight from HBM
// (Delta rows 16-byte aligned), issued before the copy so that the load overlaps it.
// Lane (c16, g) ends with U rows 4 g .. 4 g + 3 of column 16 ct + c16; column tiles
// from nv on (columns past k) keep their zero sums.
__global__ __launch_bounds__(kThreads) void write_u_mfma(FormArgs P, int64_t p0) {
  constexpr int kTiles = kMaxK / 16;
  __shared__ u32x4_t sB[2][kUSteps][kTiles][64];
  const WsLayout W = ws_layout(P.F, P.k);
  const int64_t p = p0 + blockIdx.y;
  const int64_t layer = p / P.num_chunks;
  const int j = (int)(p - layer * P.num_chunks);
  const int64_t a = min(max(P.offsets[j], (int64_t)0), P.total_tokens);
  const int64_t b = min(max(P.offsets[j + 1], a), P.total_tokens);
  const uint16_t* D = P.delta + layer * P.total_tokens * P.F;
  uint16_t* Uo = P.U_out + layer * P.total_tokens * P.m;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int m = P.m, F = P.F;
  const int nct = (m + 15) / 16;                     // column tiles of U
  const int nv = (min(m, P.k) + 15) / 16;            // column tiles of the fragments
  const int nfrag = 2 * kUSteps * nv * 64;  // fragments of one 64-feature block
  const u32x4_t* frag =
      reinterpret_cast<const u32x4_t*>(P.ws + (int64_t)blockIdx.y * W.stride + W.G);
  // t0 is uniform over the workgroup, so every thread takes the loop's barriers.
  for (int64_t t0 = a + (int64_t)blockIdx.x * 64; t0 < b; t0 += (int64_t)gridDim.x * 64) {
    f32x4_t acc[kTiles];
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int64_t trow = t0 + 16 * wave + c16;  // this lane's A row
    const bool row_ok = trow < b;
    const uint16_t* drow = D + (row_ok ? trow : a) * F + 8 * g;
    // The next 64-feature block's rows are requested before this block's fragment copy
    // and products, so their latency overlaps them (rows past the chunk read row a).
    u32x4_t avn[kUSteps];
#pragma unroll
    for (int st = 0; st < kUSteps; ++st)
      avn[st] = __builtin_nontemporal_load((const u32x4_t*)(drow + 32 * st));
    for (int f0 = 0; f0 < F; f0 += 32 * kUSteps) {  // F is a multiple of 64
      u32x4_t av[kUSteps];
#pragma unroll
      for (int st = 0; st < kUSteps; ++st) {
        av[st] = row_ok ? avn[st] : u32x4_t{0u, 0u, 0u, 0u};
        const int fn = f0 + 32 * kUSteps < F ? f0 + 32 * kUSteps : f0;
        avn[st] = __builtin_nontemporal_load((const u32x4_t*)(drow + fn + 32 * st));
      }
      const u32x4_t* src = frag + (int64_t)(f0 / 64) * nfrag;
      for (int idx = tid; idx < nfrag; idx += kThreads) {
        const int l = idx & 63, rest = idx >> 6;
        const int ct = rest % nv, q = rest / nv;  // q = part * kUSteps + step
        sB[q / kUSteps][q % kUSteps][ct][l] = src[idx];
      }
      __syncthreads();
#pragma unroll
      for (int st = 0; st < kUSteps; ++st) {
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, av[st]);
#pragma unroll
        for (int ct = 0; ct < kTiles; ++ct) {
          if (ct >= nv) break;
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              A, __builtin_bit_cast(bf16x8_t, sB[0][st][ct][lane]), acc[ct], 0, 0, 0);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              A, __builtin_bit_cast(bf16x8_t, sB[1][st][ct][lane]), acc[ct], 0, 0, 0);
        }
      }
      __syncthreads();  // the next block's copy overwrites sB
    }
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) {
      if (ct >= nct) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + 16 * wave + 4 * g + i;
        const int c = 16 * ct + c16;
        if (t < b && c < m) Uo[t * m + c] = f2bf16(acc[ct][i]);
      }
    }
  }
}

}  // namespace

int64_t form_workspace_floats(int F, int k) { return ws_layout(F, k).stride; }

namespace {
// 128 x 128 Gram tiles of problems [p0, p0 + count): rows staged by direct LDS loads
// when a chunk's rows stay below 2^31 - 64 bytes (whatever the offsets hold, a chunk
// lies inside [0, total_tokens)), else through registers.
void launch_gram128(const FormArgs& P, int64_t p0, int count, float* G, int64_t gstride,
                    hipStream_t s) {
  const int n2 = P.F / 128;
  const dim3 grid(n2 * (n2 + 1) / 2, count), blk(kThreads);
  if (P.total_tokens * P.F * 2 <= kMaxBufferBytes)
    hipLaunchKernelGGL(gram_tr, grid, blk, 0, s, P, p0, G, gstride);
  else
    hipLaunchKernelGGL(gram_tiles128, grid, blk, 0, s, P, p0, G, gstride);
}
}  // namespace

// One channel's problems [p0, p0 + count) (problem = layer * num_chunks + chunk), with
// the workspace holding `count` problems.
hipError_t launch_form_batch(const FormArgs& P, int64_t p0, int count, hipStream_t s) {
  const WsLayout W = ws_layout(P.F, P.k);
  const int F = P.F, k = P.k;
  const int nt = F / 64;
  const dim3 blk(kThreads);
  if (F % 128 == 0) {
    launch_gram128(P, p0, count, P.ws + W.G, W.stride, s);
  } else {
    hipLaunchKernelGGL(gram_tiles, dim3(nt * (nt + 1) / 2, count), blk, 0, s, P, p0,
                       P.ws + W.G, W.stride);
  }
  hipLaunchKernelGGL(init_start, dim3((F * k + kThreads - 1) / kThreads, count), blk, 0, s, P);
  const dim3 g32((k + 31) / 32, (k + 31) / 32, count);
  // Z = G Q, Q = orth(Z), `iters` + 1 times (the first from the random start).  orth is
  // Cholesky QR; the last basis gets a second pass, which restores the orthogonality
  // lost in fp32 (the iteration itself only needs the columns kept apart).  The basis
  // and the scratch columns alternate between the Q and Z regions.
  int64_t basis = W.Q, tmp = W.Z;
  auto cholqr = [&](int64_t from, int64_t to) {  // to = from R^-1
    hipLaunchKernelGGL(gram64, g32, blk, 0, s, P, from);
    hipLaunchKernelGGL(chol_rinv, dim3(count), blk, 0, s, P);
    launch_gemm_ws<false>(P, count, s, from, k, W.B, k, to, k, F, k, k);
  };
  for (int it = 0; it <= P.iters; ++it) {
    launch_gemm_ws<false>(P, count, s, W.G, F, basis, k, tmp, k, F, k, F);
    cholqr(tmp, basis);
    if (it == P.iters) {  // the basis Rayleigh-Ritz uses is orthonormalized twice
      cholqr(basis, tmp);
      const int64_t t = basis;
      basis = tmp;
      tmp = t;
    }
  }
  // Rayleigh-Ritz: tmp = G basis, B = basis^T tmp, eigenpairs of B, then tmp = basis E
  // (V_m in its first m columns).
  launch_gemm_ws<false>(P, count, s, W.G, F, basis, k, tmp, k, F, k, F);
  launch_gemm_ws<true>(P, count, s, basis, k, tmp, k, W.B, k, k, k, F);
  hipLaunchKernelGGL(jacobi_eig, dim3(count), blk, 0, s, P);
  launch_gemm_ws<false>(P, count, s, basis, k, W.E, k, tmp, k, F, k, k);
  hipLaunchKernelGGL(write_v, dim3((F * P.m + kThreads - 1) / kThreads, count), blk, 0, s, P, p0,
                     tmp);
  // Tiles of the longest chunk bound the work of one problem; the host does not read the
  // offsets, so the grid takes the average tiles per chunk (twice over, for ragged
  // chunks), or enough workgroups to fill the chip, and each workgroup loops over
  // every gx-th tile of its chunk.
  const int64_t ttiles = (P.total_tokens + 63) / 64;
  const int64_t gx = std::min<int64_t>(
      ttiles, std::max<int64_t>({(int64_t)1, 2 * ((ttiles + P.num_chunks - 1) / P.num_chunks),
                                 (2048 + count - 1) / count}));
  // U on MFMA: Delta rows are 16-byte addressable (the host requires a 16-byte aligned
  // deficit, and F is a multiple of 64).
  const int nfr = (F / 64) * kUSteps * ((std::min(P.m, k) + 15) / 16) * 64;
  hipLaunchKernelGGL(split_vm, dim3((nfr + kThreads - 1) / kThreads, count), blk, 0, s, P, tmp);
  hipLaunchKernelGGL(write_u_mfma, dim3((unsigned)gx, count), blk, 0, s, P, p0);
  return hipGetLastError();
}

// ------------------------------------------------------------------ orbit mean

namespace {

// fp64 -> bf16 bits, nearest with ties to even, as one rounding: first to fp32 with
// round-to-odd (the nearest-even fp32 value, stepped toward zero when it rounded away,
// with its last bit set when inexact), then to bf16 with ties to even.  Rounding to odd
// at 24 bits and then to nearest at 8 gives the nearest 8-bit value of x itself, since
// 24 >= 8 + 2 (in the subnormal ranges too: fp32 keeps 16 bits below bf16's quantum).
// A NaN stays a NaN (quiet); past the largest finite bf16 the result is infinity.
__device__ __forceinline__ uint16_t bf16_rne_f64(double x) {
  const float f = (float)x;
  const double back = (double)f;
  const bool inexact = back != x;
  uint32_t u = __float_as_uint(f);
  u -= (inexact && fabs(back) > fabs(x)) ? 1u : 0u;
  u |= inexact ? 1u : 0u;
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ double bf16_f64(uint32_t h) { return (double)__uint_as_float(h << 16); }

// Adds the eight bf16 values of w to acc.
__device__ __forceinline__ void add8(double (&acc)[8], const u32x4_t& w) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] += bf16_f64(w[e] & 0xffffu);
    acc[2 * e + 1] += bf16_f64(w[e] >> 16);
  }
}

// out[i] = bf16(sum_p in[p * stride + i] / num): eight values per thread and step, the
// sum in fp64 in order p = 0, 1, ..., then one division and one rounding.  HBM-bound:
// (num + 1) * 2 bytes per value.  NUM > 0: num == NUM, all of a step's loads issued
// together; NUM == 0: any num, four loads at a time.
template <int NUM>
__global__ __launch_bounds__(256) void orbit_mean_bf16(const uint16_t* in, int num, int64_t n,
                                                       int64_t stride, uint16_t* out) {
  const int64_t n8 = n >> 3;
  const int64_t step = (int64_t)gridDim.x * 256;
  if constexpr (NUM > 0) num = NUM;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n8; v += step) {
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    if constexpr (NUM > 0) {
      u32x4_t w[NUM];
#pragma unroll
      for (int p = 0; p < NUM; ++p)
        w[p] = __builtin_nontemporal_load((const u32x4_t*)(in + (int64_t)p * stride) + v);
#pragma unroll
      for (int p = 0; p < NUM; ++p) add8(acc, w[p]);
    } else {
      int p = 0;
      for (; p + 4 <= num; p += 4) {
        u32x4_t w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          w[u] = __builtin_nontemporal_load((const u32x4_t*)(in + (int64_t)(p + u) * stride) + v);
#pragma unroll
        for (int u = 0; u < 4; ++u) add8(acc, w[u]);
      }
      for (; p < num; ++p)
        add8(acc, __builtin_nontemporal_load((const u32x4_t*)(in + (int64_t)p * stride) + v));
    }
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (uint32_t)bf16_rne_f64(acc[2 * e] / (double)num) |
             ((uint32_t)bf16_rne_f64(acc[2 * e + 1] / (double)num) << 16);
    __builtin_nontemporal_store(o, (u32x4_t*)out + v);
  }
  // The last n % 8 values: one thread each in the first workgroup.
  const int64_t i = (n8 << 3) + threadIdx.x;
  if (blockIdx.x == 0 && threadIdx.x < 8 && i < n) {
    double acc = 0.0;
    for (int p = 0; p < num; ++p) acc += bf16_f64(in[(int64_t)p * stride + i]);
    out[i] = bf16_rne_f64(acc / (double)num);
  }
}

}  // namespace

hipError_t launch_orbit_mean(const uint16_t* in, int num, int64_t n, int64_t stride,
                             uint16_t* out, hipStream_t s) {
  const int64_t n8 = n >> 3;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n8 + 255) / 256, 8192));
#define KAMERA_ORBIT(N)                                                                        \
  hipLaunchKernelGGL(orbit_mean_bf16<N>, dim3((unsigned)blocks), dim3(256), 0, s, in, num, n,   \
                     stride, out)
  switch (num) {
    case 1: KAMERA_ORBIT(1); break;
    case 2: KAMERA_ORBIT(2); break;
    case 3: KAMERA_ORBIT(3); break;
    case 4: KAMERA_ORBIT(4); break;
    case 5: KAMERA_ORBIT(5); break;
    case 6: KAMERA_ORBIT(6); break;
    case 7: KAMERA_ORBIT(7); break;
    case 8: KAMERA_ORBIT(8); break;
    default: KAMERA_ORBIT(0); break;
  }
#undef KAMERA_ORBIT
  return hipGetLastError();
}

hipError_t launch_form_gram(const FormArgs& P, float* G, hipStream_t s) {
  const int nt = P.F / 64;
  const int64_t problems = (int64_t)P.num_layers * P.num_chunks;
  const int64_t gs = (int64_t)P.F * P.F;
  for (int64_t p0 = 0; p0 < problems; p0 += 65535) {
    const int count = (int)min(problems - p0, (int64_t)65535);
    if (P.F % 128 == 0) {
      launch_gram128(P, p0, count, G + p0 * gs, gs, s);
    } else {
      hipLaunchKernelGGL(gram_tiles, dim3(nt * (nt + 1) / 2, count), dim3(kThreads), 0, s, P, p0,
                         G + p0 * gs, gs);
    }
  }
  return hipGetLastError();
}

}  // namespace kamera
