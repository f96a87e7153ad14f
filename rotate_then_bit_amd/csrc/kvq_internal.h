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
  // work decomposition: an item is (tile of VPW consecutive (token, head) columns, row).
  // Two walks (set by the launcher):
  //  - tasks (rows_per_task = k > 0): one wave per (tile, run of k consecutive rows), wave
  //    w taking tile w % n_tiles and rows k * (w / n_tiles) ...; the grid holds every task.
  //  - persistent (rows_per_task = 0): W waves, as many as fit; wave w first takes tiles
  //    w, w + W, ..., w + (K-1) W (all rows of each, K = n_tiles / W), so the waves in
  //    flight cover W adjacent tiles of one row at a time; the remaining n_tiles - K W
  //    tiles are split into equal contiguous runs of (tile, row) items, one per wave.
  int64_t n_tiles;        // tiles per row
  int64_t n_items;        // rows * n_tiles
  int64_t n_waves;        // waves in the grid (set by the launcher)
  int32_t rows_per_task;  // 0: persistent walk (set by the launcher)
  int32_t trig_rows;      // RoPE table rows per wave: tokens one tile can span (set by the launcher)
  // parameters
  uint8_t perm[kMaxHeadDim];
  float quat[kMaxHeadDim / 4 * 8];
  float codebook[kMaxCodebook];
};

// Launch helpers, one per (direction, dtype, head_dim), defined in kvq_kernels.hip.
// Each returns a hipError_t as int (0 = success).
#define KVQ_DECLARE_LAUNCH(NAME) int NAME(int bits, int rot, int quant, const CodecArgs& a, void* stream);
KVQ_DECLARE_LAUNCH(launch_encode_f16_d128)
KVQ_DECLARE_LAUNCH(launch_encode_f16_d256)
KVQ_DECLARE_LAUNCH(launch_encode_bf16_d128)
KVQ_DECLARE_LAUNCH(launch_encode_bf16_d256)
KVQ_DECLARE_LAUNCH(launch_encode_f32_d128)
KVQ_DECLARE_LAUNCH(launch_encode_f32_d256)
KVQ_DECLARE_LAUNCH(launch_decode_f16_d128)
KVQ_DECLARE_LAUNCH(launch_decode_f16_d256)
KVQ_DECLARE_LAUNCH(launch_decode_bf16_d128)
KVQ_DECLARE_LAUNCH(launch_decode_bf16_d256)
KVQ_DECLARE_LAUNCH(launch_decode_f32_d128)
KVQ_DECLARE_LAUNCH(launch_decode_f32_d256)
#undef KVQ_DECLARE_LAUNCH
const char* device_error_string(int err);

}  // namespace kvq
