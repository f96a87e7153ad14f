// Internal interface between the host-side C ABI (kvq_api.cpp) and the HIP
// kernels (kvq_kernels.hip).  Not installed; callers use include/kvq.h.
#pragma once

#include <stdint.h>

namespace kvq {

constexpr int kMaxHeadDim = 256;
constexpr int kMaxCodebook = 16;
constexpr int kWavesPerBlock = 4;

// n / d for 0 <= n < 2^31 as (n * mul) >> shift, the round-up method of Granlund and
// Montgomery ("Division by invariant integers using multiplication", 1994): with
// l = ceil(log2 d), mul = floor(2^(31+l) / d) + 1 < 2^32 and shift = 31 + l.  The error
// of the product is below n * d / (d * 2^(31+l)) < 1/d, so the floor is exact.
struct FastDiv {
  uint32_t mul, shift;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while (l < 31 && (1u << l) < d) ++l;
  FastDiv f;
  f.mul = (uint32_t)((uint64_t(1) << (31 + l)) / d + 1);
  f.shift = 31 + l;
  return f;
}

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
  // work decomposition: an item is (tile of VPW consecutive (token, head) columns, row);
  // one wave per task.  Encoder task: one tile over task_len consecutive rows (wave w
  // takes tile w % n_tiles, rows from task_len * (w / n_tiles)).  Decoder task: task_len
  // consecutive tiles of one row (wave w takes tiles from task_len * (w % n_tblk), row
  // w / n_tblk).
  int64_t n_tiles;   // tiles per row (below 2^31)
  int64_t n_items;   // rows * n_tiles
  int64_t n_tblk;    // decoder: tile blocks per row (set by the launcher)
  int32_t task_len;  // set by the launcher
  FastDiv div_task;  // division by n_tiles (encoder) or n_tblk (decoder), set by the launcher
  FastDiv div_heads; // division by heads (column -> token)
  int32_t trig_rows;      // RoPE table rows per wave: tokens one tile can span (set by the launcher)
  // append (decode-step update): the input is one token per row, row r's position is
  // row_pos[r] (DEVICE), and it is written to slot row_pos[r] - pos_offset of planes with
  // cap token slots per row; NULL for a plain encode
  const int64_t* row_pos;
  int64_t cap;
  // parameters
  uint8_t perm[kMaxHeadDim];
  float quat[kMaxHeadDim / 4 * 8];
  float codebook[kMaxCodebook];
};

// Decode-step attention over an encoded cache (d = 128, Walsh-Hadamard + min-max).  The
// workspace holds the rotated queries [rows, q_heads, 128] and, per (row, query head,
// chunk of slots), a partial result: 128 rotated-domain sums, the running maximum and
// the softmax denominator.
constexpr int kAttendPart = 128 + 2;  // floats per partial
struct AttendArgs {
  const uint8_t* k_codes;
  const uint16_t* k_scale;
  const uint16_t* k_zero;
  const uint16_t* k_sink;
  const uint8_t* v_codes;
  const uint16_t* v_scale;
  const uint16_t* v_zero;
  const uint16_t* v_sink;
  const float* q;        // [rows, q_heads, 128]
  float* out;            // [rows, q_heads, 128]
  float* qrot;           // workspace: rotated queries
  float* part;           // workspace: partials [rows, q_heads, n_chunks, kAttendPart]
  const int32_t* lengths;  // DEVICE [rows] or NULL (every slot)
  int64_t rows, tokens, heads, q_heads;
  int32_t group_log2, n_sink, n_chunks, chunk;  // chunk: slots per chunk (multiple of 8)
  float scale;
  int32_t use_perm_k, use_perm_v;
  uint8_t perm_k[128];
  uint8_t perm_v[128];
};
// the chunking of the slot axis for a cache shape (same rule on both sides of the ABI).  Waves
// in flight for the partial pass: 8 K where the block-cooperative matrix-core pass runs (one
// group of 128 channels, heads a multiple of 4: measured 4.5 % faster than 16 K at the Llama-3
// cache, fewer partial rounds of resident blocks), 16 K otherwise.
inline void attend_chunks(int64_t rows, int64_t heads, int64_t tokens, bool mma_blk, int32_t* n_chunks,
                          int32_t* chunk) {
  const int64_t target = mma_blk ? 8192 : 16384;
  int64_t nc = (target + rows * heads - 1) / (rows * heads > 0 ? rows * heads : 1);
  const int64_t max_nc = (tokens + 63) / 64;
  if (nc > max_nc) nc = max_nc;
  if (nc < 1) nc = 1;
  int64_t ct = (tokens + nc - 1) / nc;
  ct = (ct + 7) / 8 * 8;
  if (ct < 8) ct = 8;
  *n_chunks = (int32_t)((tokens + ct - 1) / ct > 0 ? (tokens + ct - 1) / ct : 1);
  *chunk = (int32_t)ct;
}
int launch_attend(int bits, int qg, const AttendArgs& a, void* stream);

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
