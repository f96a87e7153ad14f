// Internal interface between the host-side C ABI (kvq_api.cpp) and the HIP
// kernels (kvq_kernels.hip).  Not installed; callers use include/kvq.h.
#pragma once

#include <stddef.h>
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
  // dynamic codebook (Lloyd-Max): dyn = 1 when on; wide_rank[j] = k for the k-th wide channel,
  // 0xff for the others; the extra plane holds the wide channels' top code bits
  int32_t dyn;
  uint8_t* extra;
  // dense rotation (DEVICE [D][D], row-major)
  const float* rot_matrix;
  // parameters
  uint8_t perm[kMaxHeadDim];
  float quat[kMaxHeadDim / 4 * 8];
  float codebook[kMaxCodebook];
  float codebook_wide[2 * kMaxCodebook];
  float chan_scale[kMaxHeadDim];
  uint8_t wide_rank[kMaxHeadDim];
};
static_assert(sizeof(CodecArgs) <= 4096, "kernel arguments above 4 KiB");

// Decode-step attention over an encoded cache (Walsh-Hadamard or no rotation + min-max).  The
// workspace holds the rotated queries [rows, q_heads, D] and, per (row, query head, chunk of
// slots), a partial result: D rotated-domain sums, the running maximum and the softmax
// denominator.  The matrix-core passes serve d = 128 with K and V alike (kAttendPart floats
// per partial); the general pass takes D + 2.
constexpr int kAttendPart = 128 + 2;  // floats per partial at d = 128
struct AttendArgs {
  const uint8_t* k_codes;
  const uint16_t* k_scale;
  const uint16_t* k_zero;
  const uint16_t* k_sink;
  const uint8_t* v_codes;
  const uint16_t* v_scale;
  const uint16_t* v_zero;
  const uint16_t* v_sink;
  const float* q;        // [rows, q_heads, D]
  float* out;            // [rows, q_heads, D]
  float* qrot;           // workspace: rotated queries
  float* part;           // workspace: partials [rows, q_heads, n_chunks, D + 2]
  const int32_t* lengths;  // DEVICE [rows] or NULL (every slot)
  int64_t rows, tokens, heads, q_heads;
  int32_t group_log2, n_sink, n_chunks, chunk;  // chunk: slots per chunk (multiple of 8)
  float scale;
  int32_t use_perm_k, use_perm_v;
  // general pass: rotation (1 Walsh-Hadamard, 0 none), V's group, and the sink slots: slots
  // 0 .. sink_slots - 1 hold the sink-plane entries sink_base .. (sink_base = pos_offset)
  int32_t rot, v_group_log2, sink_slots, sink_base;
  uint8_t perm_k[kMaxHeadDim];
  uint8_t perm_v[kMaxHeadDim];
};
// Attention entropy per (row, query head) over an encoded K cache (Walsh-Hadamard + min-max,
// head_dim 128 or 256, 2/3/4 bits): the workspace holds the rotated queries [rows, q_heads, D]
// and per (row, query head, chunk) the partial (max, sum of e^(s - max), sum of
// e^(s - max) (s - max)).
struct EntropyArgs {
  const uint8_t* k_codes;
  const uint16_t* k_scale;
  const uint16_t* k_zero;
  const uint16_t* k_sink;
  const float* q;
  float* entropy;   // [rows, q_heads]
  float* qrot;
  float* part;      // [rows, q_heads, n_chunks, 4]
  const int32_t* lengths;
  int64_t rows, tokens, heads, q_heads, head_dim;
  int32_t bits, group_log2, n_sink, n_chunks, chunk;
  float scale;
  int32_t use_perm;
  uint8_t perm[kMaxHeadDim];
};
int launch_entropy(const EntropyArgs& a, void* stream);

// The chunking of the slot axis for a cache shape (same rule on both sides of the ABI).
// Block-cooperative matrix-core pass (one group of 128 channels, heads a multiple of 4): blocks
// of 4 tasks, 3 resident per CU (168 VGPRs), 256 CUs on MI355X, so 768 blocks fill the chip
// once; the chunk count (at most 32) makes the block count the closest to whole rounds of 768,
// the fewest chunks among equals (at the Llama-3 cache, 3 chunks = one round measured 4 % faster
// than 8 chunks = 2.67 rounds, and 6 % faster than 4).  Other passes: about 16 K waves.
constexpr int64_t kAttendBlkRound = 768;
inline void attend_chunks(int64_t rows, int64_t heads, int64_t tokens, bool mma_blk, int32_t* n_chunks,
                          int32_t* chunk) {
  const int64_t max_nc = (tokens + 63) / 64;
  int64_t nc = 1;
  if (mma_blk) {
    const int64_t quads = rows * heads / 4 > 0 ? rows * heads / 4 : 1;
    double best = -1.0;
    for (int64_t k = 1; k <= 32 && k <= max_nc; ++k) {
      const double rounds = (double)(quads * k) / (double)kAttendBlkRound;
      const double whole = rounds <= 1.0 ? 1.0 : __builtin_ceil(rounds);
      const double eff = rounds / whole;
      if (eff > best + 1e-9) {
        best = eff;
        nc = k;
      }
    }
  } else {
    const int64_t target = 16384;
    nc = (target + rows * heads - 1) / (rows * heads > 0 ? rows * heads : 1);
    if (nc > max_nc) nc = max_nc;
  }
  if (nc < 1) nc = 1;
  int64_t ct = (tokens + nc - 1) / nc;
  ct = (ct + 7) / 8 * 8;
  if (ct < 8) ct = 8;
  *n_chunks = (int32_t)((tokens + ct - 1) / ct > 0 ? (tokens + ct - 1) / ct : 1);
  *chunk = (int32_t)ct;
}
int launch_attend(int bits, int qg, const AttendArgs& a, void* stream);
// the general pass (any configuration check_attend admits); one translation unit per
// (head_dim, K bits)
int launch_attend_gen_d128_k2(int v_bits, int qg, const AttendArgs& a, void* stream);
int launch_attend_gen_d128_k3(int v_bits, int qg, const AttendArgs& a, void* stream);
int launch_attend_gen_d128_k4(int v_bits, int qg, const AttendArgs& a, void* stream);
int launch_attend_gen_d256_k2(int v_bits, int qg, const AttendArgs& a, void* stream);
int launch_attend_gen_d256_k3(int v_bits, int qg, const AttendArgs& a, void* stream);
int launch_attend_gen_d256_k4(int v_bits, int qg, const AttendArgs& a, void* stream);
// The allocation-free attention entry point keeps its workspace in a static device array of
// this many bytes (one copy per GPU, held until the process ends).
constexpr size_t kAttendScratchBytes = size_t(32) << 20;
// Device address of that array on the current device (looked up once per device with
// hipGetSymbolAddress); returns a hipError_t as int.
int attend_scratch(void** ptr);

// Calibration of the RotateKV variants: per-channel statistics of a calibration slice (for the
// outlier-aware permutation) and activation-based sink detection.
struct CalibArgs {
  const void* x;  // [R, T, H, D] with strides (elements)
  int64_t rows, tokens, heads, head_dim;
  int64_t sr, st, sh;
  int64_t pos_offset;
  double rope_log2_base;
  int32_t dtype, rope, n_sink;
  int32_t tpw;       // tokens per wave of the statistics pass
  int64_t n_waves;   // waves of the statistics pass: rows * ceil(tokens / tpw)
  double* part;      // workspace [n_waves, D]: per-wave sums of |y_c|
  double* stats;     // [D]: mean |y_c| over the non-sink vectors
  double lambda;     // sink threshold (times the row's lower median token norm)
  double* norms;     // [R, T] token norms
  uint8_t* flags;    // [R, T]
  int32_t* counts;   // [R]
  int32_t* prefix;   // [R]: one past the last flagged token (0 if none)
  double* medians;   // [R] lower median token norm
  // rotated moments (dynamic codebook): the codec's front end on each vector
  int32_t rot, use_perm;
  const float* rot_matrix;       // DEVICE [D][D] (dense rotation)
  uint8_t perm[kMaxHeadDim];
  float quat[kMaxHeadDim / 4 * 8];
};
inline int32_t calib_tokens_per_wave(int64_t rows, int64_t tokens) {
  // about 8 K waves over the slice, at least 16 tokens each
  const int64_t want = (rows * tokens + 8191) / 8192;
  const int64_t t = ((want > 16 ? want : 16) + 15) / 16 * 16;
  return (int32_t)(t > (1 << 20) ? (1 << 20) : t);
}
int launch_channel_stats(const CalibArgs& a, void* stream);
int launch_detect_sinks(const CalibArgs& a, void* stream);
int launch_rotated_moments(const CalibArgs& a, void* stream);

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
// The dense rotation (head_dim 128; dtype / out_dtype: DT_F16, DT_BF16, DT_F32), and its sink pass.
int launch_encode_dense(int dtype, int bits, int quant, const CodecArgs& a, void* stream);
int launch_decode_dense(int out_dtype, int bits, int quant, const CodecArgs& a, void* stream);
const char* device_error_string(int err);

}  // namespace kvq
