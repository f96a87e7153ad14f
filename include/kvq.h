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
 * between calls except a thread-local error message.  The caller owns every
 * buffer.  Calls only enqueue work on the given HIP stream and never
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

#define KVQ_ABI_VERSION 1

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
  KVQ_ERR_UNSUPPORTED = 8, /* head_dim not in {128, 256}                               */
  KVQ_ERR_ABI = 9,         /* cfg->abi_version != KVQ_ABI_VERSION                      */
  KVQ_ERR_DEVICE = 10,     /* the HIP runtime refused the launch (message has detail)  */
  KVQ_ERR_INTERNAL = 11
} kvq_status;

/* Element types (enum values are stored as int32_t in the structs below). */
typedef enum kvq_dtype { KVQ_F16 = 0, KVQ_BF16 = 1, KVQ_F32 = 2 } kvq_dtype;
typedef enum kvq_rot { KVQ_ROT_NONE = 0, KVQ_ROT_FWHT = 1, KVQ_ROT_SO4 = 2 } kvq_rot;
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
} kvq_config;

/* Packed planes, all DEVICE pointers, 16-byte aligned, contiguous, row-major:
 *   codes [R,T,H,D*bits/8] u8     -- always
 *   scale [R,T,H,D/G]      fp16   -- min-max only
 *   zero  [R,T,H,D/G]      fp16   -- min-max only
 *   norm  [R,T,H]          fp32   -- Lloyd-Max only (rho)
 *   sink  [R,n_sink,H,D]   fp16   -- when n_sink > 0; slot p holds position p.
 * Planes a configuration does not use may be NULL.  Sink vectors have all-zero
 * codes, scale, zero and norm slots. */
typedef struct kvq_planes {
  void* codes;
  void* scale;
  void* zero;
  void* norm;
  void* sink;
} kvq_planes;

/* KVQ_ABI_VERSION of the loaded library. */
int32_t kvq_abi_version(void);

/* Host-only: check a configuration (no device access). */
kvq_status kvq_validate(const kvq_config* cfg);

/* Host-only: byte sizes of the five planes for cfg (0 for planes it does not use). */
kvq_status kvq_packed_sizes(const kvq_config* cfg, size_t* codes_bytes, size_t* scale_bytes,
                            size_t* zero_bytes, size_t* norm_bytes, size_t* sink_bytes);

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
 * cached values).  The keys are never decoded: with the orthonormal Hadamard rotation M and
 * the keys' permutation P, q . k_t = (M P q) . y_t for the stored y_t = zero + code * scale,
 * and the values are summed in the rotated domain and rotated back once per output (the
 * rotation of the RotateKV page, whose decode-stage speed-up this serves).  Sink slots are
 * read from the fp16 sink planes.  Scores and sums are fp32; for 2-bit codes with one group
 * of 128 channels the products run exactly on the int8 matrix cores, with the rotated query
 * rounded to 2^-31 of 16 times its largest element and each softmax weight to 2^-27 of the
 * largest weight x value scale of its 128-slot window.
 *   cfg_k, cfg_v  the K and V caches: same rows R, slots T, heads H, head_dim 128, bits
 *                 (2 or 4), group (32, 64 or 128), n_sink (at most 64), Walsh-Hadamard and
 *                 min-max, pos_offset 0 (slot t holds position t); each its own permutation
 *                 and RoPE flag (keys hold post-RoPE values; q must be rotated by RoPE at its
 *                 own position by the caller).  Otherwise KVQ_ERR_UNSUPPORTED / KVQ_ERR_SHAPE.
 *   k, v          DEVICE planes of the two caches (as written by kvq_encode / kvq_append).
 *   q, out        DEVICE float32 [R, q_heads, 128], contiguous; q_heads = H * g, g in {1, 2, 4}.
 *   lengths       DEVICE int32 [R]: slots each row attends over (clamped to [0, T]); NULL = T.
 *                 A row with no slot gets zeros.
 *   scale         score multiplier (head_dim^-1/2 in the page's code); finite.
 *   workspace     DEVICE, 16-byte aligned, at least kvq_attend_workspace_size(cfg_k, q_heads)
 *                 bytes, owned by the caller; its contents are scratch between calls.
 * Asynchronous; calls that share a workspace must not overlap. */
kvq_status kvq_attend_workspace_size(const kvq_config* cfg_k, int64_t q_heads, size_t* bytes);
kvq_status kvq_attend(const kvq_config* cfg_k, const kvq_planes* k, const kvq_config* cfg_v, const kvq_planes* v,
                      const float* q, int64_t q_heads, const int32_t* lengths, float scale, float* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Decode in's planes into y (DEVICE, contiguous [R,T,H,D] of y_dtype).  Asynchronous.
 * y must not alias any plane. */
kvq_status kvq_decode(const kvq_config* cfg, const kvq_planes* in, void* y, int32_t y_dtype,
                      void* stream);

/* Host-only: Lloyd-Max codebook (2^bits ascending levels) for N(0, sigma^2), written
 * to codebook_out as float32; the classical fixed point of midpoint thresholds and
 * conditional-mean levels, iterated in double precision (IsoQuant page, section 3.1
 * names the Lloyd-Max quantizer; the fitting procedure is the textbook one). */
kvq_status kvq_lloyd_max_gaussian(int32_t bits, double sigma, float* codebook_out);

/* Static description of a status code. */
const char* kvq_status_string(kvq_status status);

/* Detail of the last error on the calling thread ("" if none). */
const char* kvq_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
