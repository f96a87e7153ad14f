/*
 * kvq -- rotation + low-bit codec for KV-cache vectors on AMD MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; no framework types.  Link with
 * librotate_then_bit_amd's libkvq.so (built by the package's build script).
 *
 * What it computes, per token-head vector x of a [rows, tokens, heads, head_dim]
 * tensor at position p = pos_offset + t (references are to the pages this codec
 * is written from; see the repository's design notes for the full list):
 *
 *   1. RoPE (optional, keys): pairs (2i, 2i+1) rotated by p * base^(-2i/d)
 *      -- EliteKV page, section 2.1 (rotation matrix R_m); RoPE-KV page, section 1.
 *   2. Attention sinks: positions p < n_sink are stored as fp16 of the post-RoPE
 *      vector and skip the rest -- RotateKV page (attention-sink-aware quantization).
 *   3. Norm separation (Lloyd-Max only): rho = |x|, u = x / (rho + 1e-6)
 *      -- IsoQuant page, section 3.1 step 1.
 *   4. Channel permutation (optional): u'[j] = u[perm[j]]
 *      -- RotateKV page (outlier-aware rotation by channel reordering).
 *   5. Rotation: Walsh-Hadamard z = H u / sqrt(d) (RotateKV page), or per 4-D
 *      block z_b = qL_b * u_b * qR_b with unit quaternions (IsoQuant page,
 *      sections 2.2 and 3.2), or none.
 *   6. Quantization to 2/3/4 bits: per-group asymmetric min-max with fp16
 *      zero = round-down(min) and scale = round-up((max - zero)/(2^b - 1)),
 *      q = rint((z - zero)/scale); or Lloyd-Max, q = #{k : z > (c_k + c_{k+1})/2}
 *      -- IsoQuant page, section 3.1 step 2.
 *   7. Bit-packing, LSB first: bit m of code j is bit b*j + m of the vector's stream.
 *
 * Decoding is the inverse (IsoQuant page, section 3.1 step 3): unpack,
 * dequantize, inverse rotation, inverse permutation, times rho; sink positions
 * return their fp16 values.  There is no inverse RoPE: the output is the
 * post-RoPE key a cache holds.
 *
 * Threading and memory: the library allocates nothing and keeps no state
 * between calls except a thread-local error message and the static device
 * workspace of kvq_attend_noalloc.  The caller owns every other buffer.  Calls only enqueue work on the given HIP stream and never
 * synchronise; buffers must stay alive until that work completes.  All
 * argument checking happens on the host before anything is enqueued, so a
 * call that returns an error has done nothing.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 4

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_NULL = 1,        /* a required pointer is NULL                              */
  KVQ_ERR_SHAPE = 2,       /* negative size, size overflow or invalid strides          */
  KVQ_ERR_BITS = 3,        /* bits not in {2, 3, 4}                                    */
  KVQ_ERR_GROUP = 4,       /* min-max group size not in {32,64,128,256} or not | d     */
  KVQ_ERR_ROT = 5,         /* unknown rotation / quantizer / dtype enum value          */
  KVQ_ERR_PARAM = 6,       /* perm not a permutation, quaternion not unit, codebook
                              not finite and strictly ascending, bad rope base or
                              position range                                          */
  KVQ_ERR_ALIGN = 7,       /* a device pointer or stride is not 16-byte aligned        */
  KVQ_ERR_UNSUPPORTED = 8, /* head_dim not in {128, 256}, or a combination not built   */
  KVQ_ERR_ABI = 9,         /* cfg->abi_version != KVQ_ABI_VERSION                      */
  KVQ_ERR_DEVICE = 10,     /* the HIP runtime refused the launch (message has detail)  */
  KVQ_ERR_INTERNAL = 11
} kvq_status;

/* Element types (enum values are stored as int32_t in the structs below). */
typedef enum kvq_dtype { KVQ_F16 = 0, KVQ_BF16 = 1, KVQ_F32 = 2 } kvq_dtype;
typedef enum kvq_rot { KVQ_ROT_NONE = 0, KVQ_ROT_FWHT = 1, KVQ_ROT_SO4 = 2, KVQ_ROT_DENSE = 3, KVQ_ROT_ROTOR = 4 } kvq_rot;
typedef enum kvq_quant { KVQ_Q_MINMAX = 0, KVQ_Q_LLOYD = 1 } kvq_quant;

typedef struct kvq_config {
  int32_t abi_version;  /* = KVQ_ABI_VERSION                                          */
  int32_t dtype;        /* kvq_dtype of the encode input x                            */
  int64_t rows;         /* R: batch rows (e.g. layers x batch folded together)        */
  int64_t tokens;       /* T: token positions                                         */
  int64_t heads;        /* H: KV heads, at most 32768                                 */
  int64_t head_dim;     /* D: 128 or 256                                              */
  int64_t stride_r;     /* encode-input strides in ELEMENTS; D is always contiguous.  */
  int64_t stride_t;     /*   all three 0 = contiguous [R,T,H,D].  Each must be a      */
  int64_t stride_h;     /*   multiple of 16 bytes' worth of elements.                 */
  int32_t bits;         /* 2, 3 or 4                                                  */
  int32_t group_size;   /* min-max group of contiguous rotated channels: 32, 64, 128,
                           256, dividing D (ignored by Lloyd-Max)                     */
  int32_t quant;        /* kvq_quant                                                  */
  int32_t rot;          /* kvq_rot                                                    */
  int32_t rope;         /* 1: apply RoPE before anything else                         */
  int32_t n_sink;       /* positions p < n_sink are stored as fp16 sinks (>= 0)       */
  double rope_base;     /* RoPE base, e.g. 10000.0 (must be > 1 when rope = 1)        */
  int64_t pos_offset;   /* position of token 0; 0 <= pos_offset, pos_offset + T <= 2^31 */
  const uint16_t* perm;     /* HOST [D] gather map u'[j] = u[perm[j]], or NULL         */
  const float* quat;        /* HOST [D/4][2][4]: (qL, qR) per block, each (w,x,y,z),
                               unit norm within 1e-4; required for KVQ_ROT_SO4         */
  const float* codebook;    /* HOST [2^bits] strictly ascending, finite; required for
                               KVQ_Q_LLOYD                                             */
  /* Dynamic codebook (IsoQuant page, section 4.2), Lloyd-Max only; all NULL = off.  Rotated
   * channel j is quantized against codebook scaled by chan_scale[j]; the head_dim/16 channels
   * with chan_wide[j] = 1 use codebook_wide (twice the levels) scaled the same way, the top bit
   * of their bits+1-bit code going to the extra plane.  kvq_dynamic_codebook derives all three
   * from kvq_rotated_moments. */
  const float* chan_scale;    /* HOST [D], finite and > 0                                 */
  const uint8_t* chan_wide;   /* HOST [D], 0 or 1, exactly D/16 ones                       */
  const float* codebook_wide; /* HOST [2^(bits+1)] strictly ascending, finite              */
  /* KVQ_ROT_DENSE: DEVICE [D][D] float32 row-major, z_i = sum_j M[i][j] u_j; orthogonal (a
   * precondition the host cannot check: decode applies the transpose).  The baselines the
   * IsoQuant page, section 1, compares against: a dense random rotation (TurboQuant), or
   * 3-D rotors as a block-diagonal matrix (RotorQuant, kvq_rotor_matrix).  Codec (encode,
   * decode): head_dim 128, no dynamic codebook; not in append or attention. */
  const float* rot_matrix;
  /* KVQ_ROT_ROTOR: RotorQuant's 3-D rotors (IsoQuant page, section 1), computed as rotors:
   * channels 3b .. 3b + 2 (b < D / 3) turn by the sandwich product rotor_quat[b] (0, v)
   * rotor_quat[b]* (section 2.1); a 2-channel tail (D mod 3 = 2) turns in its plane by
   * rotor_tail radians; a 1-channel tail stays.  Codec (encode, decode) only. */
  const float* rotor_quat;  /* HOST [D/3][4] (w, x, y, z), unit norm within 1e-4             */
  double rotor_tail;        /* finite                                                       */
} kvq_config;

/* Packed planes, all DEVICE pointers, 16-byte aligned, contiguous, row-major:
 *   codes [R,T,H,D*bits/8] u8     -- always
 *   scale [R,T,H,D/G]      fp16   -- min-max only
 *   zero  [R,T,H,D/G]      fp16   -- min-max only
 *   norm  [R,T,H]          fp32   -- Lloyd-Max only (rho)
 *   sink  [R,n_sink,H,D]   fp16   -- when n_sink > 0; slot p holds position p.
 *   extra [R,T,H,D/128]    u8     -- dynamic codebook only: bit k (LSB first) is the top
 *                                    code bit of the k-th wide channel (increasing order)
 * Planes a configuration does not use may be NULL.  Sink vectors have all-zero
 * codes, scale, zero, norm and extra slots. */
typedef struct kvq_planes {
  void* codes;
  void* scale;
  void* zero;
  void* norm;
  void* sink;
  void* extra;
} kvq_planes;

/* KVQ_ABI_VERSION of the loaded library. */
int32_t kvq_abi_version(void);

/* Host-only: check a configuration (no device access). */
kvq_status kvq_validate(const kvq_config* cfg);

/* Host-only: byte sizes of the six planes for cfg (0 for planes it does not use). */
kvq_status kvq_packed_sizes(const kvq_config* cfg, size_t* codes_bytes, size_t* scale_bytes,
                            size_t* zero_bytes, size_t* norm_bytes, size_t* sink_bytes, size_t* extra_bytes);

/* Encode x (DEVICE, dtype cfg->dtype, [R,T,H,D] with cfg's strides) into out's planes.
 * stream: a hipStream_t (NULL = the default stream).  Asynchronous.  x must not
 * alias any plane.  Sink slots for positions outside [pos_offset, pos_offset+T) are
 * left untouched. */
kvq_status kvq_encode(const kvq_config* cfg, const void* x, const kvq_planes* out, void* stream);

/* Decode-step append: encode one new token per row into an encoded cache, as the
 * cache update of single-token decoding does (EliteKV page, section 7.1: each step's
 * post-RoPE key and value are appended at the sequence's current length).
 *   cfg        describes the CACHE: rows R, tokens = T slots per row (slot s holds
 *              position pos_offset + s), heads, head_dim, dtype of x, bits, rotation,
 *              quantizer, RoPE, sinks and parameters exactly as for kvq_encode.
 *   x          DEVICE, dtype cfg->dtype: one vector per (row, head), element (r, h, c) at
 *              x + r*stride_r + h*stride_h + c (stride_t is not used; all strides 0 =
 *              contiguous [R, H, D]).
 *   positions  DEVICE int64 [R]: the position of row r's new token.  The token is encoded
 *              exactly as kvq_encode encodes a token at that position (its RoPE angle; a
 *              sink, i.e. fp16 into sink slot positions[r] with zeroed code, scale, zero
 *              and norm slots, when positions[r] < n_sink) and written to slot
 *              positions[r] - pos_offset of every plane of that row.  A row whose position
 *              lies outside [pos_offset, pos_offset + T) writes nothing.
 *   cache      DEVICE planes of the [R, T, H] cache, laid out as for kvq_encode.  Slots
 *              other than the written ones are not touched.
 * Asynchronous; x must not alias any plane.  The positions are read on the device, so
 * they are not checked on the host beyond the pointer (a row with an out-of-range
 * position is skipped, as above). */
kvq_status kvq_append(const kvq_config* cfg, const void* x, const int64_t* positions, const kvq_planes* cache,
                      void* stream);

/* Decode-step attention over an encoded K/V cache: for every row r and query head m,
 *   out[r, m] = sum_t softmax_t(scale * q[r, m] . k_t) v_t   over slots t < lengths[r],
 * where k_t, v_t are the cache's decoded vectors (what kvq_decode returns) of KV head
 * m / (q_heads / heads) -- the attention of the EliteKV page, section 7.1 (query scaled,
 * scored against the cached post-RoPE keys, softmax over positions, weighted sum of the
 * cached values).  The keys are never decoded: with the orthonormal rotation M (Hadamard /
 * sqrt(head_dim), or the identity for an unrotated cache) and the keys' permutation P,
 * q . k_t = (M P q) . y_t for the stored y_t = zero + code * scale, and the values are summed
 * in the rotated domain and rotated back once per output (the rotation of the RotateKV page,
 * whose decode-stage speed-up this serves).  Slots whose position (pos_offset + slot) is
 * below n_sink are read from the fp16 sink planes.  Scores and sums are fp32.  For head_dim
 * 128, Walsh-Hadamard, K and V of equal bits (2 or 4) and group, pos_offset 0 and at most 4
 * query heads per KV head, the products run on the int8 matrix cores, exactly for 2-bit
 * codes with one group of 128 channels (the rotated query rounded to 2^-31 of 16 times its
 * largest element and each softmax weight to 2^-27 of the largest weight x value scale of
 * its 128-slot window); every other supported cache takes a vector-ALU pass.
 *   cfg_k, cfg_v  the K and V caches: same rows R, slots T, heads H, head_dim (128 or 256),
 *                 n_sink (at most 64), pos_offset, rotation (Walsh-Hadamard or none) and
 *                 min-max quantizer; each its own bits (2, 3 or 4), group, permutation and
 *                 RoPE flag (keys hold post-RoPE values; q must be rotated by RoPE at its
 *                 own position by the caller).  Otherwise KVQ_ERR_UNSUPPORTED / KVQ_ERR_SHAPE.
 *   k, v          DEVICE planes of the two caches (as written by kvq_encode / kvq_append).
 *   q, out        DEVICE float32 [R, q_heads, head_dim], contiguous; q_heads = H * g,
 *                 g in {1, 2, 4, 8}.
 *   lengths       DEVICE int32 [R]: slots each row attends over (clamped to [0, T]); NULL = T.
 *                 A row with no slot gets zeros.
 *   scale         score multiplier (head_dim^-1/2 in the page's code); finite.
 *   workspace     DEVICE, 16-byte aligned, at least kvq_attend_workspace_size(cfg_k, cfg_v,
 *                 q_heads) bytes, owned by the caller; its contents are scratch between calls.
 * Asynchronous; calls that share a workspace must not overlap.
 * kvq_attend_workspace_size: the workspace a call with these caches needs (cfg_v NULL: a V
 * cache configured like cfg_k); the same checks as kvq_attend on the configurations. */
kvq_status kvq_attend_workspace_size(const kvq_config* cfg_k, const kvq_config* cfg_v, int64_t q_heads,
                                     size_t* bytes);
kvq_status kvq_attend(const kvq_config* cfg_k, const kvq_planes* k, const kvq_config* cfg_v, const kvq_planes* v,
                      const float* q, int64_t q_heads, const int32_t* lengths, float scale, float* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free variant of kvq_attend, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments, results and errors are those of kvq_attend without the workspace: the
 * workspace is instead a static device array inside the library, of
 * kvq_attend_noalloc_max_workspace() bytes (32 MiB; one copy on each GPU the library runs
 * on, held until the process ends; its device address is looked up on the first call on
 * each device).  A cache and query-head count whose kvq_attend_workspace_size exceeds that
 * returns KVQ_ERR_SHAPE before anything is enqueued.  The call allocates nothing.
 * Every call on one GPU uses that GPU's one array: calls that overlap on a GPU (on
 * different streams, or from different threads) race and give wrong results; serialise
 * them.  The array keeps the last call's contents; no call relies on them (every byte a
 * call reads was written by that call). */
kvq_status kvq_attend_noalloc(const kvq_config* cfg_k, const kvq_planes* k, const kvq_config* cfg_v,
                              const kvq_planes* v, const float* q, int64_t q_heads, const int32_t* lengths, float scale,
                              float* out, void* stream);
size_t kvq_attend_noalloc_max_workspace(void);

/* Decode in's planes into y (DEVICE, contiguous [R,T,H,D] of y_dtype).  Asynchronous.
 * y must not alias any plane. */
kvq_status kvq_decode(const kvq_config* cfg, const kvq_planes* in, void* y, int32_t y_dtype,
                      void* stream);

/* Calibration of the outlier-aware channel reordering (RotateKV page, method summary and key
 * design: channel reordering adapts the Walsh-Hadamard rotation to the channel-wise outlier
 * distribution).  Reads a calibration slice x exactly as kvq_encode would (cfg's shape, dtype,
 * strides, RoPE, positions; sink positions p < n_sink are left out) and writes
 *   stats    DEVICE double [head_dim]: mean |y_c| over every non-sink vector, y the post-RoPE
 *            vector (the input itself without RoPE); 0 for an empty slice.
 *   workspace DEVICE, 8-byte aligned, at least kvq_channel_stats_workspace_size(cfg) bytes
 *            (per-wave float64 sums; scratch between calls).
 * Sums are float64, in a fixed order (deterministic).  Asynchronous. */
kvq_status kvq_channel_stats_workspace_size(const kvq_config* cfg, size_t* bytes);
kvq_status kvq_channel_stats(const kvq_config* cfg, const void* x, double* stats, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Host-only: the outlier-aware gather map perm (HOST uint16 [head_dim], for kvq_config.perm)
 * from per-channel statistics (HOST double [head_dim], e.g. kvq_channel_stats copied back).
 * The head_dim / group_size channels with the largest statistic go to positions 0, G, 2G, ...
 * (largest first; equal statistics in increasing channel order); the other channels fill the
 * remaining positions in increasing order.  After the Sylvester-ordered Walsh-Hadamard
 * transform a channel at a multiple of G enters every coefficient of a min-max group with the
 * same sign, so it shifts the group (absorbed by its zero) without widening its range. */
kvq_status kvq_outlier_perm(const double* stats, int64_t head_dim, int32_t group_size, uint16_t* perm);

/* Activation-based attention-sink detection (RotateKV page: attention-sink-aware
 * quantization identifies the sinks from their massive activations).  For every row r and
 * token t of x (read as kvq_encode reads it; RoPE does not change a norm):
 *   norms[r, t]  DEVICE double [R, T]: L2 norm of the token over all heads and channels
 *                (squares summed in float64, exact for 16-bit inputs);
 *   medians[r]   DEVICE double [R]: the row's lower median norm (rank floor((T-1)/2));
 *   flags[r, t]  DEVICE uint8 [R, T]: 1 where norms[r, t] > lambda * medians[r];
 *   counts[r]    DEVICE int32 [R]: flagged tokens; prefix[r] DEVICE int32 [R]: one past the
 *                last flagged token (0 if none) -- the n_sink that keeps every detected sink
 *                of the row in the codec's fp16 sink slots.
 * lambda: finite, >= 0.  Asynchronous. */
kvq_status kvq_detect_sinks(const kvq_config* cfg, const void* x, double lambda, double* norms, uint8_t* flags,
                            int32_t* counts, int32_t* prefix, double* medians, void* stream);

/* Dynamic codebook calibration (IsoQuant page, section 4.2: per-channel statistics gathered
 * online, KL-optimised boundaries, a codebook twice the size for outlier channels).
 * kvq_rotated_moments runs the codec's front end (RoPE, norm separation u = y/(rho + 1e-6),
 * permutation, rotation; cfg->quant must be KVQ_Q_LLOYD) on every non-sink vector of the
 * calibration slice x and writes
 *   moments    DEVICE double [D]: mean z_j^2 per rotated channel j;
 *   workspace  DEVICE, 8-byte aligned, at least kvq_channel_stats_workspace_size(cfg) bytes.
 * Asynchronous; float64 sums in a fixed order. */
kvq_status kvq_rotated_moments(const kvq_config* cfg, const void* x, double* moments, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Host-only: the dynamic codebook from the moments (HOST double [D], each > 0):
 * chan_scale[j] = sqrt(moments[j]) -- the zero-mean Gaussian closest to channel j in KL
 * divergence has its second moment; chan_wide: 1 on the D/16 channels with the largest
 * moments (equal moments in increasing channel order); codebook and codebook_wide: the
 * Lloyd-Max codebooks of N(0, 1) with 2^bits and 2^(bits+1) levels.  All outputs HOST
 * arrays of D, D, 2^bits and 2^(bits+1) entries, ready for kvq_config. */
kvq_status kvq_dynamic_codebook(const double* moments, int64_t head_dim, int32_t bits, float* chan_scale,
                                uint8_t* chan_wide, float* codebook, float* codebook_wide);

/* Dynamic bit width (IsoQuant page, section 6.2: each head's attention entropy, widths in
 * proportion, the quantization kernel of each width).  kvq_attention_entropy writes
 *   entropy  DEVICE float [R, q_heads]: the entropy (nats) of the softmax attention of q[r, m]
 *            over the first lengths[r] slots of the K cache (as kvq_attend scores them:
 *            scale * q . k, keys in the rotated domain, sinks from the fp16 planes); 0 for a
 *            row with no slot.
 * cfg_k: Walsh-Hadamard + min-max, head_dim 128 or 256, 2/3/4 bits, any group, pos_offset 0;
 * q DEVICE float [R, q_heads, D] contiguous, q_heads = heads * g, g in {1, 2, 4, 8}; lengths
 * DEVICE int32 [R] or NULL; workspace DEVICE, 16-byte aligned, at least
 * kvq_attention_entropy_workspace_size bytes.  Asynchronous. */
kvq_status kvq_attention_entropy_workspace_size(const kvq_config* cfg_k, int64_t q_heads, size_t* bytes);
kvq_status kvq_attention_entropy(const kvq_config* cfg_k, const kvq_planes* k, const float* q, int64_t q_heads,
                                 const int32_t* lengths, float scale, float* entropy, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Host-only: per-head widths bits[h] in [lo, hi] (2 <= lo <= hi <= 4) summing to total, in
 * proportion to entropy[h] (HOST double [heads], each finite >= 0; e.g. the mean of
 * kvq_attention_entropy over rows and the query heads of KV head h): the share
 * total * e_h / sum(e) floored into [lo, hi], then one bit at a time to the largest remainder
 * (lowest head first) while short, off the smallest remainder (highest head first) while over.
 * Each head is then encoded at its width (a head shard through the stride arguments). */
kvq_status kvq_allocate_bits(const double* entropy, int64_t heads, int32_t total, int32_t lo, int32_t hi,
                             int32_t* bits);

/* Host-only: Lloyd-Max codebook (2^bits ascending levels, bits 1..5) for N(0, sigma^2), written
 * to codebook_out as float32; the classical fixed point of midpoint thresholds and
 * conditional-mean levels, iterated in double precision (IsoQuant page, section 3.1
 * names the Lloyd-Max quantizer; the fitting procedure is the textbook one). */
kvq_status kvq_lloyd_max_gaussian(int32_t bits, double sigma, float* codebook_out);

/* Host-only: RotorQuant's rotation (the 3-D Clifford rotors the IsoQuant page, section 1,
 * compares against) as the matrix of a KVQ_ROT_DENSE rotation: the block-diagonal [D][D]
 * float32 row-major matrix whose block b (rows and columns 3b .. 3b + 2, b < D / 3) maps v to
 * the vector part of rq[b] (0, v) rq[b]* (the sandwich product of section 2.1, written out
 * as the 3x3 matrix of the quaternion), whose 2-channel tail (D mod 3 = 2) turns in its plane
 * by tail_angle, and whose 1-channel tail (D mod 3 = 1) is left as it is.
 *   rq          HOST float32 [D / 3][4], (w, x, y, z), each of unit norm within 1e-4.
 *   head_dim    128 or 256 (the dense codec takes 128).
 *   out         HOST float32 [D][D], written whole; owned by the caller.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_UNSUPPORTED (head_dim), KVQ_ERR_PARAM (a quaternion off unit
 * norm or not finite, tail_angle not finite). */
kvq_status kvq_rotor_matrix(const float* rq, int64_t head_dim, float tail_angle, float* out);

/* Static description of a status code. */
const char* kvq_status_string(kvq_status status);

/* Detail of the last error on the calling thread ("" if none). */
const char* kvq_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
