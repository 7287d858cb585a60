// Internal interface between the host ABI (abi.cpp) and the gfx950 kernels (kernels.hip).
#pragma once
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace kamera {

constexpr int kMaxTunedHalf = 64;     // tuned kernels rotate at most 128 dims per head
constexpr int kMaxBlockTokens = 512;  // tokens one tuned workgroup covers, at most
// The rotate+patch kernel addresses one layer of a channel (and one layer of U) through
// a buffer resource with 32-bit byte offsets; byte offset 2^31 is its "no row" value,
// so every range it covers ends at or below this.
constexpr int64_t kMaxBufferBytes = ((int64_t)1 << 31) - 64;

// One channel as the kernels see it.  Pointers are device pointers; strides are in
// elements of the storage type.
struct ChanArgs {
  void* data;
  int64_t layer_stride, slot_stride, head_stride, page_stride;
  // Out-of-place destination (recall): whole result rows go here, through its own
  // strides and the destination block table.  nullptr: in place.
  void* out;
  int64_t out_layer_stride, out_slot_stride, out_head_stride, out_page_stride;
  const void* U;  // [layers][tokens][rank]
  const void* V;  // [layers][chunks][heads*dim][rank]
  const float* scale;  // fp8 E4M3: [layers] dequantisation scales; else unused
  // rotate+patch kernel: bytes one layer spans (largest element offset + 1, times the
  // element size) in the source, the destination and U.
  uint32_t layer_bytes, out_layer_bytes, u_layer_bytes;
  int32_t heads, dim, rope_dim;
  int32_t fblocks;   // rotate+patch kernel: 128-feature blocks per token row
  int64_t blocks;    // tuned kernels: workgroups of this channel per layer
  // Pair frequencies theta^(-2i/rope_dim), i < rope_dim/2, formed on the host in fp64.
  double omega[kMaxTunedHalf];
};

struct CommonArgs {
  const int64_t* offsets;   // [chunks + 1]
  const int64_t* delta;     // [chunks]
  const int32_t* block_table;
  int64_t total_tokens;
  int64_t num_pages;
  int64_t token_groups;     // ceil(total_tokens / block_tokens)
  double theta;
  int32_t num_chunks;
  int32_t page_size;
  int32_t num_layers;
  int32_t rank;
  int32_t block_tokens;     // tokens one workgroup covers (tuned kernels)
  int32_t page_shift;       // log2(page_size) when it is a power of two, else -1
  int32_t tail_mode;        // rotate+patch tail launch: 1 by boundary, 2 by token group
  int32_t dtype;            // storage type: 0 bf16, 1 fp32, 2 fp8 E4M3 (factors bf16)
  // Positional variant: pairing 0 = NeoX half-split (i, i + r/2), 1 = interleaved
  // (2i, 2i + 1); delta holds num_sections values per chunk (M-RoPE when > 1), and
  // rotary pair i belongs to the first section s with i < sec_end[s].
  int32_t pairing;
  int32_t num_sections;
  int32_t sec_end[4];
  // Pool order (rotate+patch in place over one chunk of a paged cache): inv[p] is the
  // logical page that pool page p holds, -1 for none; pool_slots = num_pages * page_size.
  const int32_t* inv;
  int64_t num_logical_pages;
  int64_t pool_slots;
  // Destination paging (out of place only).
  const int32_t* out_block_table;
  int64_t out_num_pages;
  int32_t out_page_size;
  int32_t out_page_shift;
};

// Patch formation for one channel: top-m factors of each (layer, chunk) deficit.
struct FormArgs {
  const uint16_t* delta;    // [layers][total_tokens][F] bf16
  const int64_t* offsets;   // [num_chunks + 1]
  float* ws;                // workspace of the current batch
  uint16_t* U_out;          // [layers][total_tokens][m] bf16
  uint16_t* V_out;          // [layers][num_chunks][F][m] bf16
  float* sigma_out;         // [layers][num_chunks][m] or nullptr
  int64_t total_tokens;
  int32_t num_chunks;
  int32_t F;                // feature width, a multiple of 64, at most 1024
  int32_t k;                // subspace width: min(m + 16, F, 128), even
  int32_t m;
  int32_t iters;            // subspace iterations after the first
  int32_t num_layers;
};

// Relocate-on-read decode attention (attend.hip): K = channel 0, V = channel 1, bf16,
// dim 128, rank a multiple of 8 up to 128.  The workspace holds the prepared queries
// (qw: [layers][chunks][num_q_heads][128 + rank]: the rotated query and V_K^T q, both
// times scale * log2 e) and the partial slots (ws: [layers][num_q_heads][slots]
// [slot_floats]: max, sum, chunk index, 128 value sums, rank U_V sums).  Tokens are cut
// into `splits` ranges of `split_tokens`, and each range into segments at chunk
// boundaries; segment (split s, chunk j) writes slot s + j.  Slots no segment writes
// keep the zero sum the prep kernel stores.
struct AttendArgs {
  const void* data[2];
  int64_t layer_stride[2], slot_stride[2], head_stride[2], page_stride[2];
  const void* U[2];           // [layers][tokens][rank] bf16, or nullptr at rank 0
  const void* V[2];           // [layers][chunks][heads*128][rank] bf16
  const int32_t* block_table;
  int64_t num_pages;
  const int64_t* offsets;     // [chunks + 1]
  const int64_t* delta;       // [chunks][num_sections]
  const float* q;             // [layers][num_q_heads][128]
  float* out;                 // [layers][num_q_heads][128]
  float* lse;                 // [layers][num_q_heads] or nullptr
  float* qw;                  // prepared queries (see above)
  float* ws;                  // partial slots (see above)
  int64_t total_tokens;
  int32_t num_chunks, num_sections, sec_end[4], pairing, rope_dim;
  int32_t page_size, num_layers, heads, num_q_heads, group, rank;
  int32_t splits, split_tokens, slots, slot_floats;
  uint32_t layer_bytes[2];    // bytes of one layer of each channel (below 2^31 - 64)
  int32_t double_buffer;      // tile kernel: the next tile's V rows go to a second LDS tile
  int32_t fp8;                // KV elements are fp8 E4M3 codes with per-layer scales
  int32_t heads_mapping;      // tile kernel: one wave per KV head, a workgroup per range
  const float* kv_scale[2];   // fp8: [layers] scale of K and of V; else nullptr
  float scale_log2;           // softmax scale * log2(e): scores are kept in base 2
  double omega[64];           // theta^(-2i/rope_dim)
};

constexpr int kAttendDim = 128;
constexpr int kAttendMaxGroup = 8;
constexpr int kAttendMaxHeadsPerGroup = 8;
// Compute units of the part (MI355X): the attention planner sizes one round of
// one-wave-per-KV-head workgroups by it.
constexpr int kAttendCus = 256;  // KV heads of the one-wave-per-head mapping
// Floats of one partial slot at rank m: max, sum, chunk, one unused float (the sums
// start 16-byte aligned), 128 value sums, m U_V sums; padded to a multiple of 4.
constexpr int kAttendSlotHead = 4;
constexpr int attend_slot_floats(int m) { return (kAttendSlotHead + kAttendDim + m + 3) & ~3; }

hipError_t launch_attend(const AttendArgs& a, hipStream_t s);

// Floats of workspace one problem needs.
int64_t form_workspace_floats(int F, int k);
// Problems [p0, p0 + count) of one channel (problem = layer * num_chunks + chunk).
hipError_t launch_form_batch(const FormArgs& a, int64_t p0, int count, hipStream_t s);
// Gram matrices of every problem of one channel into G [problems][F][F].
hipError_t launch_form_gram(const FormArgs& a, float* G, hipStream_t s);
// Orbit deficit: out[i] = bf16(sum_p in[p * stride + i] / num), fp64 sum and division,
// one rounding (in, out 16-byte aligned, stride a multiple of 8).
hipError_t launch_orbit_mean(const uint16_t* in, int num, int64_t n, int64_t stride,
                             uint16_t* out, hipStream_t s);

// Rotation only, bf16 (16-byte accesses) or fp8 (8-byte accesses): rope_dim in
// {16, 32, 64, 128}.  `unroll` row groups per wavefront (bf16: 2 or 4; fp8: 4 or 8).
hipError_t launch_rotate_rows(const ChanArgs& ch, const CommonArgs& cm, int unroll,
                              hipStream_t s);

// Rotation + rank-m patch on MFMA, bf16 or fp8 (fp8: rank % 8 == 0):
// see kernels.hip for the shape conditions.
// With ChanArgs::out set it runs out of place (rank % 8 == 0; rank 0 allowed).
// Covers nch (1 or 2) channels in one launch, plus a second launch for the token groups
// that chunk boundaries cut when there is more than one chunk.
// valu: the head launch of a bf16 in-place call with rank <= 64 (a multiple of 8) takes
// the patch on VALU instead of MFMA (a measurement variant).
// pool: sweep a paged cache in pool order through cm.inv (in place, one chunk, page size a
// multiple of 16; channel blocks counted over cm.pool_slots); no tail launch.
hipError_t launch_relocate_patch_rows(const ChanArgs* ch, int nch, const CommonArgs& cm,
                                      int valu, bool pool, hipStream_t s);

// inv[p] = the index k of the block-table entry that names pool page p (entries outside
// [0, num_pages) name none), -1 for pool pages no entry names; inv has num_pages entries.
// Two launches: fill, then scatter (entries are pairwise distinct by precondition).
hipError_t launch_table_inverse(const int32_t* table, int64_t entries, int64_t num_pages,
                                int32_t* inv, hipStream_t s);

// Pool pages whose inverse table fits the library-held scratch array (4 MiB per GPU).
constexpr int64_t kScratchPoolPages = (int64_t)1 << 20;
// Device address of the scratch array on the GPU that `s` belongs to (looked up once per
// GPU; no allocation).
hipError_t scratch_inverse_table(hipStream_t s, int32_t** out);

// Plain per-row kernel: any dim, even rope_dim, rank <= KAMERA_MAX_RANK, bf16, fp32 or
// fp8, element-aligned pointers.  In place with rank 0 it only touches rotated dims; out of
// place (ChanArgs::out set) it writes whole rows.
hipError_t launch_generic(const ChanArgs& ch, const CommonArgs& cm, int dtype, hipStream_t s);

}  // namespace kamera
