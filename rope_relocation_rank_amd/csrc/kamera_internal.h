// Internal interface between the host ABI (abi.cpp) and the gfx950 kernels (kernels.hip).
#pragma once
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace kamera {

// One channel as the kernels see it.  Pointers are device pointers; strides are in
// elements of the storage type.
struct ChanArgs {
  void* data;
  int64_t layer_stride, slot_stride, head_stride, page_stride;
  const void* U;  // [layers][tokens][rank]
  const void* V;  // [layers][chunks][heads*dim][rank]
  int32_t heads, dim, rope_dim;
  int32_t tasks_per_head;  // rotate+patch kernel: dim / 64
  int32_t groups;          // rotate+patch kernel: ceil(heads * tasks_per_head / tasks_per_wave)
  int32_t pad_;
  int64_t units;           // wavefront units of this channel per layer
};

struct CommonArgs {
  const int64_t* offsets;   // [chunks + 1]
  const int64_t* delta;     // [chunks]
  const int32_t* block_table;
  int64_t total_tokens;
  int64_t num_pages;
  int64_t nranges;          // ceil(total_tokens / range_tokens)
  double theta;
  int32_t num_chunks;
  int32_t page_size;
  int32_t num_layers;
  int32_t rank;
  int32_t range_tokens;     // tokens per wavefront unit (multiple of 16)
  int32_t pad_;
};

// Rotation only, bf16, 16-byte rows: half = rope_dim / 2 in {8, 16, 32, 64, 128}.
hipError_t launch_rotate_bf16(const ChanArgs& ch, const CommonArgs& cm, hipStream_t s);

// Rotation + rank-m patch with MFMA, bf16: dim % 64 == 0, rope_dim % 64 == 0, rank <= 128.
// Covers nch (1 or 2) channels in one launch.
hipError_t launch_relocate_patch_mfma(const ChanArgs* ch, int nch, const CommonArgs& cm,
                                      int tasks_per_wave, hipStream_t s);

// Plain per-row kernel: any dim, even rope_dim, rank <= KAMERA_MAX_RANK, bf16 or fp32,
// element-aligned pointers.  With rank 0 it only touches rotated dims.
hipError_t launch_generic(const ChanArgs& ch, const CommonArgs& cm, int dtype, hipStream_t s);

}  // namespace kamera
