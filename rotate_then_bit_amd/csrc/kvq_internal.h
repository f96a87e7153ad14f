// Internal interface between the host-side C ABI (kvq_api.cpp) and the HIP
// kernels (kvq_kernels.hip).  Not installed; callers use include/kvq.h.
#pragma once

#include <stdint.h>

namespace kvq {

constexpr int kMaxHeadDim = 256;
constexpr int kMaxCodebook = 16;
constexpr int kWavesPerBlock = 4;

// Everything a kernel needs, passed by value in the kernel-argument segment
// (about 2.6 KB), so no device allocation is ever made for parameters.
struct CodecArgs {
  // device buffers
  const void* x;       // encode input (strided) / unused by decode
  void* y;             // decode output (contiguous) / unused by encode
  uint8_t* codes;
  uint16_t* scale;
  uint16_t* zero;
  float* norm;
  uint16_t* sink;
  // shape
  int64_t rows, tokens, heads;
  int64_t sr, st, sh;  // encode-input strides in elements
  int64_t pos_offset;
  double rope_log2_base;
  int32_t group_log2;
  int32_t n_sink;
  int32_t rope;
  int32_t use_perm;
  // work decomposition: items = n_tiles * n_row_chunks, one wave per item
  int32_t rows_per_item;
  int32_t n_tiles;
  int32_t n_row_chunks;
  int32_t xcd_remap;
  // parameters
  uint8_t perm[kMaxHeadDim];
  float quat[kMaxHeadDim / 4 * 8];
  float codebook[kMaxCodebook];
};

// Launch helpers, one per (direction, dtype), defined in kvq_kernels.hip.
// Each returns a hipError_t as int (0 = success).
#define KVQ_DECLARE_LAUNCH(NAME) \
  int NAME(int head_dim, int bits, int rot, int quant, const CodecArgs& a, void* stream);
KVQ_DECLARE_LAUNCH(launch_encode_f16)
KVQ_DECLARE_LAUNCH(launch_encode_bf16)
KVQ_DECLARE_LAUNCH(launch_encode_f32)
KVQ_DECLARE_LAUNCH(launch_decode_f16)
KVQ_DECLARE_LAUNCH(launch_decode_bf16)
KVQ_DECLARE_LAUNCH(launch_decode_f32)
#undef KVQ_DECLARE_LAUNCH
const char* device_error_string(int err);

}  // namespace kvq
