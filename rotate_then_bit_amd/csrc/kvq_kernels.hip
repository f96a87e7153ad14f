// HIP kernels of the rotation + low-bit KV-cache codec, written for gfx950 (CDNA4).
//
// Work layout.  A sub-wavefront of LV = D/32 lanes owns one token-head vector
// (LV = 4 at d = 128, 8 at d = 256), so a wave64 holds VPW = 64/LV vectors.
// Each lane holds 32 elements as 4 chunks of 8 consecutive channels; chunk k of
// lane l covers channels e = (k*LV + l)*8 + s, s = 0..7.  This interleave makes
// every 16-byte load or store of a 16-bit tensor coalesced across the wave
// (VPW consecutive vectors are 16*VPW*LV contiguous bytes per instruction).
//
// A wave processes a tile of VPW consecutive (token, head) columns for a
// range of rows; RoPE angles depend only on the column, so they are computed
// once per tile and kept in registers across the rows.
//
// Walsh-Hadamard: the channel index bits split into in-lane bits (s and k) and
// lane bits (l).  In-lane butterflies are plain VALU adds; lane-bit butterflies
// use a DPP-fused v_fmac (partner * m + own) for lane xor 1/2 and ds_swizzle for
// xor 4.  The fmac form leaves lanes with a set bit holding the negated value;
// the sign after all lane stages is (-1)^popcount(l) and is folded into the
// quantization scale (encode) or the output scale (decode).
//
// LDS holds only parameters (RoPE frequencies, SO(4) matrices, the Lloyd-Max
// codebook) and, when a channel permutation is used, a per-wave scratch through
// which the permutation is applied (a gather of 32 values per lane).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

enum { DT_F16 = 0, DT_BF16 = 1, DT_F32 = 2 };
enum { ROT_NONE = 0, ROT_FWHT = 1, ROT_SO4 = 2 };
enum { Q_MINMAX = 0, Q_LLOYD = 1 };

constexpr int kNC = 4;  // 8-element chunks per lane (32 elements per lane)

template <int D>
struct Geo {
  static constexpr int LV = D / 32;                 // lanes per vector
  static constexpr int LVB = (LV == 4) ? 2 : 3;      // log2(LV)
  static constexpr int VPW = 64 / LV;                // vectors per wave
  static constexpr int STRIDE = D + 4;               // floats per vector in the perm scratch
};

// ---------------------------------------------------------------------------
// cross-lane primitives
// ---------------------------------------------------------------------------
#define KVQ_QP1 " quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
#define KVQ_QP2 " quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"

// v <- partner(v) * m + v for 8 values, partner = lane xor 1.  The leading
// s_nop covers the VALU-write -> DPP-read hazard on the first operand.
__device__ __forceinline__ void fmac_x1(float* v, float m) {
  asm("s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %8" KVQ_QP1 "\n\t"
      "v_fmac_f32_dpp %1, %1, %8" KVQ_QP1 "\n\t"
      "v_fmac_f32_dpp %2, %2, %8" KVQ_QP1 "\n\t"
      "v_fmac_f32_dpp %3, %3, %8" KVQ_QP1 "\n\t"
      "v_fmac_f32_dpp %4, %4, %8" KVQ_QP1 "\n\t"
      "v_fmac_f32_dpp %5, %5, %8" KVQ_QP1 "\n\t"
      "v_fmac_f32_dpp %6, %6, %8" KVQ_QP1 "\n\t"
      "v_fmac_f32_dpp %7, %7, %8" KVQ_QP1
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
        "+v"(v[7])
      : "v"(m));
}

__device__ __forceinline__ void fmac_x2(float* v, float m) {
  asm("s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %8" KVQ_QP2 "\n\t"
      "v_fmac_f32_dpp %1, %1, %8" KVQ_QP2 "\n\t"
      "v_fmac_f32_dpp %2, %2, %8" KVQ_QP2 "\n\t"
      "v_fmac_f32_dpp %3, %3, %8" KVQ_QP2 "\n\t"
      "v_fmac_f32_dpp %4, %4, %8" KVQ_QP2 "\n\t"
      "v_fmac_f32_dpp %5, %5, %8" KVQ_QP2 "\n\t"
      "v_fmac_f32_dpp %6, %6, %8" KVQ_QP2 "\n\t"
      "v_fmac_f32_dpp %7, %7, %8" KVQ_QP2
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
        "+v"(v[7])
      : "v"(m));
}

__device__ __forceinline__ float swz_x4(float v) {
  // ds_swizzle bit mode: and 0x1f, or 0, xor 4
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F));
}

__device__ __forceinline__ float min_x1(float v) {
  asm("s_nop 1\n\tv_min_f32_dpp %0, %0, %0" KVQ_QP1 : "+v"(v));
  return v;
}
__device__ __forceinline__ float min_x2(float v) {
  asm("s_nop 1\n\tv_min_f32_dpp %0, %0, %0" KVQ_QP2 : "+v"(v));
  return v;
}
__device__ __forceinline__ float max_x1(float v) {
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0" KVQ_QP1 : "+v"(v));
  return v;
}
__device__ __forceinline__ float max_x2(float v) {
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0" KVQ_QP2 : "+v"(v));
  return v;
}
__device__ __forceinline__ float add_x1(float v) {
  asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0" KVQ_QP1 : "+v"(v));
  return v;
}
__device__ __forceinline__ float add_x2(float v) {
  asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0" KVQ_QP2 : "+v"(v));
  return v;
}

// Sum / max over the LV lanes of a vector.
template <int LV>
__device__ __forceinline__ float vec_sum(float v) {
  v = add_x1(v);
  v = add_x2(v);
  if constexpr (LV == 8) v += swz_x4(v);
  return v;
}
template <int LV>
__device__ __forceinline__ float vec_max(float v) {
  v = max_x1(v);
  v = max_x2(v);
  if constexpr (LV == 8) v = fmaxf(v, swz_x4(v));
  return v;
}

// ---------------------------------------------------------------------------
// Walsh-Hadamard, unnormalised, on the 32 values of a lane plus the lane bits.
// On return lane l holds (-1)^popcount(l) times the true coefficients.
// ---------------------------------------------------------------------------
template <int LV>
__device__ __forceinline__ void fwht_lane(float* v, int l) {
  // slot bits (s = 0..7 within each chunk)
#pragma unroll
  for (int hb = 1; hb < 8; hb <<= 1) {
#pragma unroll
    for (int k = 0; k < kNC; ++k) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s & hb) continue;
        float a = v[8 * k + s], b = v[8 * k + s + hb];
        v[8 * k + s] = a + b;
        v[8 * k + s + hb] = a - b;
      }
    }
  }
  // chunk bits (k = 0..3)
#pragma unroll
  for (int hk = 1; hk < kNC; hk <<= 1) {
#pragma unroll
    for (int k = 0; k < kNC; ++k) {
      if (k & hk) continue;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        float a = v[8 * k + s], b = v[8 * (k + hk) + s];
        v[8 * k + s] = a + b;
        v[8 * (k + hk) + s] = a - b;
      }
    }
  }
  // lane bits
  const float m1 = (l & 1) ? -1.0f : 1.0f;
  const float m2 = (l & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int k = 0; k < kNC; ++k) fmac_x1(v + 8 * k, m1);
#pragma unroll
  for (int k = 0; k < kNC; ++k) fmac_x2(v + 8 * k, m2);
  if constexpr (LV == 8) {
    const float m4 = (l & 4) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(swz_x4(v[i]), m4, v[i]);
  }
}

__device__ __forceinline__ float lane_sign(int l) {
  return (__builtin_popcount(l) & 1) ? -1.0f : 1.0f;
}

// ---------------------------------------------------------------------------
// dtype conversions
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ void load_chunk(const void* base, int64_t off, float* v) {
  if constexpr (DT == DT_F32) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == DT_BF16) {
        v[2 * i] = __uint_as_float(ws[i] << 16);
        v[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
      } else {
        v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws[i] & 0xffffu));
        v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws[i] >> 16));
      }
    }
  }
}

__device__ __forceinline__ uint32_t f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

template <int DT>
__device__ __forceinline__ void store_chunk(void* base, int64_t off, const float* v) {
  if constexpr (DT == DT_F32) {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + off);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint32_t ws[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == DT_BF16)
        ws[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
      else
        ws[i] = f16_bits(v[2 * i]) | (f16_bits(v[2 * i + 1]) << 16);
    }
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(base) + off) =
        make_uint4(ws[0], ws[1], ws[2], ws[3]);
  }
}

// fp16 with directed rounding, from the IEEE bit pattern of the nearest value.
__device__ __forceinline__ uint32_t f16_round_down(float x) {
  _Float16 h = (_Float16)x;
  uint32_t b = __builtin_bit_cast(uint16_t, h);
  if ((float)h > x) b = (b & 0x8000u) ? b + 1u : (b == 0u ? 0x8001u : b - 1u);
  return b;
}
__device__ __forceinline__ uint32_t f16_round_up(float x) {
  _Float16 h = (_Float16)x;
  uint32_t b = __builtin_bit_cast(uint16_t, h);
  if ((float)h < x) b = (b & 0x8000u) ? (b == 0x8000u ? 0x0001u : b - 1u) : b + 1u;
  return b;
}
__device__ __forceinline__ float f16_value(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// ---------------------------------------------------------------------------
// bit-packing of one chunk (8 codes, 8*BITS bits, byte offset chunk*BITS)
// ---------------------------------------------------------------------------
template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t* rec, int chunk, uint32_t word) {
  if constexpr (BITS == 2) {
    *reinterpret_cast<uint16_t*>(rec + 2 * chunk) = (uint16_t)word;
  } else if constexpr (BITS == 4) {
    *reinterpret_cast<uint32_t*>(rec + 4 * chunk) = word;
  } else {
    uint8_t* p = rec + 3 * chunk;
    if ((chunk & 1) == 0) {
      *reinterpret_cast<uint16_t*>(p) = (uint16_t)word;
      p[2] = (uint8_t)(word >> 16);
    } else {
      p[0] = (uint8_t)word;
      *reinterpret_cast<uint16_t*>(p + 1) = (uint16_t)(word >> 8);
    }
  }
}

template <int BITS>
__device__ __forceinline__ uint32_t load_codes(const uint8_t* rec, int chunk) {
  if constexpr (BITS == 2) {
    return *reinterpret_cast<const uint16_t*>(rec + 2 * chunk);
  } else if constexpr (BITS == 4) {
    return *reinterpret_cast<const uint32_t*>(rec + 4 * chunk);
  } else {
    const uint8_t* p = rec + 3 * chunk;
    if ((chunk & 1) == 0)
      return (uint32_t)*reinterpret_cast<const uint16_t*>(p) | ((uint32_t)p[2] << 16);
    return (uint32_t)p[0] | ((uint32_t)*reinterpret_cast<const uint16_t*>(p + 1) << 8);
  }
}

// ---------------------------------------------------------------------------
// parameter staging shared by both kernels
// ---------------------------------------------------------------------------
// SO(4) block matrix M = L(qL) R(qR): M v = qL * v * qR (Hamilton product, real first).
__device__ void build_so4(const float* q, float* m) {
  const float aw = q[0], ax = q[1], ay = q[2], az = q[3];
  const float bw = q[4], bx = q[5], by = q[6], bz = q[7];
  const float L[16] = {aw, -ax, -ay, -az, ax, aw, -az, ay, ay, az, aw, -ax, az, -ay, ax, aw};
  const float R[16] = {bw, -bx, -by, -bz, bx, bw, bz, -by, by, -bz, bw, bx, bz, by, -bx, bw};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) acc = __builtin_fmaf(L[4 * i + k], R[4 * k + j], acc);
      m[4 * i + j] = acc;
    }
}

// cos/sin of the RoPE angle phi = pos * theta, evaluated in double precision:
// quadrant reduction phi = k*pi/2 + r, |r| <= pi/4 (two-term Cody-Waite split of
// pi/2, exact products for k < 2^31), then the Taylor series of sin and cos in r
// (terms up to r^17 / r^16, truncation error < 1e-17), rounded once to float.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, double theta, float* c, float* s) {
  constexpr double kTwoOverPi = 0.63661977236758138;
  constexpr double kPio2Hi = 1.570796012878418;       // pi/2 truncated to 22 bits
  constexpr double kPio2Lo = 3.139164786504813e-07;   // pi/2 - kPio2Hi (rounded)
  const double phi = (double)pos * theta;
  const double k = rint(phi * kTwoOverPi);
  double r = fma(-k, kPio2Hi, phi);
  r = fma(-k, kPio2Lo, r);
  const double r2 = r * r;
  // sin r = r (1 - r2/3! + r2^2/5! - ...), cos r = 1 - r2/2! + r2^2/4! - ...
  double sn = 1.0 / 355687428096000.0;                   // 1/17!
  sn = fma(sn, -r2, 1.0 / 1307674368000.0);              // 1/15!
  sn = fma(sn, -r2, 1.0 / 6227020800.0);
  sn = fma(sn, -r2, 1.0 / 39916800.0);
  sn = fma(sn, -r2, 1.0 / 362880.0);
  sn = fma(sn, -r2, 1.0 / 5040.0);
  sn = fma(sn, -r2, 1.0 / 120.0);
  sn = fma(sn, -r2, 1.0 / 6.0);
  sn = fma(sn, -r2, 1.0);
  sn *= r;
  double cs = 1.0 / 20922789888000.0;                    // 1/16!
  cs = fma(cs, -r2, 1.0 / 87178291200.0);                // 1/14!
  cs = fma(cs, -r2, 1.0 / 479001600.0);                  // 1/12!
  cs = fma(cs, -r2, 1.0 / 3628800.0);                    // 1/10!
  cs = fma(cs, -r2, 1.0 / 40320.0);                      // 1/8!
  cs = fma(cs, -r2, 1.0 / 720.0);                        // 1/6!
  cs = fma(cs, -r2, 1.0 / 24.0);                         // 1/4!
  cs = fma(cs, -r2, 0.5);                                // 1/2!
  cs = fma(cs, -r2, 1.0);
  const int quad = (int)((int64_t)k & 3);
  double oc, os;
  switch (quad) {
    case 0: oc = cs; os = sn; break;
    case 1: oc = -sn; os = cs; break;
    case 2: oc = -cs; os = -sn; break;
    default: oc = sn; os = -cs; break;
  }
  *c = (float)oc;
  *s = (float)os;
}

// ---------------------------------------------------------------------------
// ENCODE
// ---------------------------------------------------------------------------
template <int DT, int D, int BITS, int ROT, int QUANT>
__global__ void __launch_bounds__(64 * kWavesPerBlock) encode_kernel(const CodecArgs a) {
  using G = Geo<D>;
  constexpr int LV = G::LV, VPW = G::VPW;
  extern __shared__ float s_scratch[];
  __shared__ double s_theta[D / 2];
  __shared__ float s_mat[ROT == ROT_SO4 ? (D / 4) * 16 : 1];

  const int tid = threadIdx.x;
  if (a.rope) {
    for (int i = tid; i < D / 2; i += blockDim.x)
      s_theta[i] = exp2(-(2.0 * (double)i / (double)D) * a.rope_log2_base);
  }
  if constexpr (ROT == ROT_SO4) {
    for (int b = tid; b < D / 4; b += blockDim.x) build_so4(&a.quat[8 * b], &s_mat[16 * b]);
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  int64_t block = blockIdx.x;
  if (a.xcd_remap) {
    const int64_t nb = gridDim.x;
    block = (block & 7) * (nb >> 3) + (block >> 3);
  }
  const int64_t item = block * kWavesPerBlock + wave;
  if (item >= (int64_t)a.n_tiles * a.n_row_chunks) return;  // wave-uniform; no barrier follows

  const int tile = (int)(item % a.n_tiles);
  const int rc = (int)(item / a.n_tiles);
  const int q = lane / LV, l = lane % LV;
  const int64_t ncols = a.tokens * a.heads;
  const int64_t col = (int64_t)tile * VPW + q;
  const bool valid = col < ncols;
  const int64_t t = valid ? col / a.heads : 0;
  const int64_t h = valid ? col - t * a.heads : 0;
  const int64_t pos = a.pos_offset + t;
  const bool is_sink = valid && pos < a.n_sink;
  const bool work = valid && !is_sink;
  const int64_t r0 = (int64_t)rc * a.rows_per_item;
  const int64_t r1 = min(a.rows, r0 + a.rows_per_item);
  const int64_t xoff = t * a.st + h * a.sh;

  // RoPE angles for this lane's 16 channel pairs (fixed across rows)
  float rc_[16], rs_[16];
  if (a.rope) {
#pragma unroll
    for (int k = 0; k < kNC; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = (k * LV + l) * 4 + j;
        rope_cos_sin(pos, s_theta[i], &rc_[4 * k + j], &rs_[4 * k + j]);
      }
  }

  // permutation gather addresses (bytes within the wave's scratch)
  float* scratch = s_scratch + wave * VPW * G::STRIDE;
  int paddr[32];
  if (a.use_perm) {
#pragma unroll
    for (int k = 0; k < kNC; ++k)
#pragma unroll
      for (int s = 0; s < 8; ++s)
        paddr[8 * k + s] = q * G::STRIDE + (int)a.perm[(k * LV + l) * 8 + s];
  }

  const float norm_c = (ROT == ROT_FWHT) ? (float)(1.0 / __builtin_sqrt((double)D)) : 1.0f;
  const float sgn = (ROT == ROT_FWHT) ? lane_sign(l) : 1.0f;
  const int gb = a.group_log2;
  const int LB = (QUANT == Q_MINMAX) ? min(G::LVB, gb - 3) : 0;     // lane bits inside a group
  const int CB = (QUANT == Q_MINMAX) ? max(0, gb - 3 - G::LVB) : 0; // chunk bits inside a group
  const int64_t ngroups = (QUANT == Q_MINMAX) ? (D >> gb) : 0;

  for (int64_t r = r0; r < r1; ++r) {
    const int64_t vec = r * ncols + col;  // index into the packed planes
    float v[32];
    if (valid) {
#pragma unroll
      for (int k = 0; k < kNC; ++k) load_chunk<DT>(a.x, r * a.sr + xoff + (k * LV + l) * 8, v + 8 * k);
      if (a.rope) {
#pragma unroll
        for (int k = 0; k < kNC; ++k)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x0 = v[8 * k + 2 * j], x1 = v[8 * k + 2 * j + 1];
            const float c = rc_[4 * k + j], s = rs_[4 * k + j];
            v[8 * k + 2 * j] = __builtin_fmaf(x0, c, -x1 * s);
            v[8 * k + 2 * j + 1] = __builtin_fmaf(x0, s, x1 * c);
          }
      }
    }
    if (is_sink) {
      const int64_t srow = (r * a.n_sink + pos) * a.heads + h;
#pragma unroll
      for (int k = 0; k < kNC; ++k) store_chunk<DT_F16>(a.sink, srow * D + (k * LV + l) * 8, v + 8 * k);
      uint8_t* rec = a.codes + vec * (D * BITS / 8);
#pragma unroll
      for (int k = 0; k < kNC; ++k) store_codes<BITS>(rec, k * LV + l, 0u);
      if constexpr (QUANT == Q_MINMAX) {
        for (int g = l; g < ngroups; g += LV) {
          a.scale[vec * ngroups + g] = 0;
          a.zero[vec * ngroups + g] = 0;
        }
      } else {
        if (l == 0) a.norm[vec] = 0.0f;
      }
    }
    if (work) {
      if constexpr (QUANT == Q_LLOYD) {
        // |x| with an exact power-of-two pre-scale by the largest |x_i|, so that the
        // sum of squares neither underflows nor overflows in float
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
        amax = vec_max<LV>(amax);
        const int ex = (amax > 0.0f) ? __builtin_amdgcn_frexp_expf(amax) : 0;
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const float w = __builtin_ldexpf(v[i], -ex);
          ss = __builtin_fmaf(w, w, ss);
        }
        ss = vec_sum<LV>(ss);
        const float rho = __builtin_ldexpf(__builtin_sqrtf(ss), ex);
        const float inv = 1.0f / (rho + 1e-6f);
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] *= inv;
        if (l == 0) a.norm[vec] = rho;
      }
      if (a.use_perm) {
        // natural order in, gathered order out (one wave, in-order LDS)
#pragma unroll
        for (int k = 0; k < kNC; ++k) {
          float4* dst = reinterpret_cast<float4*>(scratch + q * G::STRIDE + (k * LV + l) * 8);
          dst[0] = make_float4(v[8 * k], v[8 * k + 1], v[8 * k + 2], v[8 * k + 3]);
          dst[1] = make_float4(v[8 * k + 4], v[8 * k + 5], v[8 * k + 6], v[8 * k + 7]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = scratch[paddr[i]];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      if constexpr (ROT == ROT_FWHT) {
        fwht_lane<LV>(v, l);
      } else if constexpr (ROT == ROT_SO4) {
#pragma unroll
        for (int k = 0; k < kNC; ++k)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int blk = (k * LV + l) * 2 + half;
            const float* m = &s_mat[16 * blk];
            float* u = v + 8 * k + 4 * half;
            const float u0 = u[0], u1 = u[1], u2 = u[2], u3 = u[3];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              u[i] = __builtin_fmaf(m[4 * i], u0,
                     __builtin_fmaf(m[4 * i + 1], u1, __builtin_fmaf(m[4 * i + 2], u2, m[4 * i + 3] * u3)));
          }
      }
      const float A = sgn * norm_c;  // true coefficient = A * v
      uint8_t* rec = a.codes + vec * (D * BITS / 8);
      if constexpr (QUANT == Q_MINMAX) {
        float cmn[kNC], cmx[kNC];
#pragma unroll
        for (int k = 0; k < kNC; ++k) {
          float lo = v[8 * k], hi = v[8 * k];
#pragma unroll
          for (int s = 1; s < 8; ++s) {
            lo = fminf(lo, v[8 * k + s]);
            hi = fmaxf(hi, v[8 * k + s]);
          }
          // true values are A * v
          cmn[k] = (A > 0.0f) ? lo * A : hi * A;
          cmx[k] = (A > 0.0f) ? hi * A : lo * A;
        }
        if (CB >= 1) {
#pragma unroll
          for (int k = 0; k < kNC; k += 2) {
            cmn[k] = cmn[k + 1] = fminf(cmn[k], cmn[k + 1]);
            cmx[k] = cmx[k + 1] = fmaxf(cmx[k], cmx[k + 1]);
          }
        }
        if (CB >= 2) {
          cmn[0] = cmn[1] = cmn[2] = cmn[3] = fminf(cmn[0], cmn[2]);
          cmx[0] = cmx[1] = cmx[2] = cmx[3] = fmaxf(cmx[0], cmx[2]);
        }
        // per-group zero/scale: reduce over the group's lanes, round to fp16
        // (zero down, scale up), store from the group's first lane
        auto group = [&](float mn, float mx, int k, float& zo, float& io) {
          if (LB >= 1) { mn = min_x1(mn); mx = max_x1(mx); }
          if (LB >= 2) { mn = min_x2(mn); mx = max_x2(mx); }
          if (LB >= 3) { mn = fminf(mn, swz_x4(mn)); mx = fmaxf(mx, swz_x4(mx)); }
          // "+ 0.0f" turns a -0 (all-zero group, negated lanes) into +0
          const uint32_t zb = f16_round_down(mn + 0.0f);
          const float z = f16_value(zb);
          const uint32_t sb = f16_round_up((mx - z) / (float)((1 << BITS) - 1) + 0.0f);
          const float sc = f16_value(sb);
          if ((l & ((1 << LB) - 1)) == 0) {
            const int64_t gi = ((int64_t)((k * LV + l) * 8)) >> gb;
            a.scale[vec * ngroups + gi] = (uint16_t)sb;
            a.zero[vec * ngroups + gi] = (uint16_t)zb;
          }
          zo = z;
          io = (sc > 0.0f) ? 1.0f / sc : 0.0f;
        };
        float zf[kNC], inv[kNC];
        group(cmn[0], cmx[0], 0, zf[0], inv[0]);
        if (CB == 0) {
          group(cmn[1], cmx[1], 1, zf[1], inv[1]);
          group(cmn[2], cmx[2], 2, zf[2], inv[2]);
          group(cmn[3], cmx[3], 3, zf[3], inv[3]);
        } else if (CB == 1) {
          group(cmn[2], cmx[2], 2, zf[2], inv[2]);
          zf[1] = zf[0]; inv[1] = inv[0];
          zf[3] = zf[2]; inv[3] = inv[2];
        } else {
          zf[1] = zf[2] = zf[3] = zf[0];
          inv[1] = inv[2] = inv[3] = inv[0];
        }
#pragma unroll
        for (int k = 0; k < kNC; ++k) {
          const float z = zf[k], iv = inv[k];
          uint32_t word = 0;
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            float tq = (__builtin_fmaf(v[8 * k + s], A, -z)) * iv;
            tq = fminf(fmaxf(__builtin_rintf(tq), 0.0f), (float)((1 << BITS) - 1));
            word |= ((uint32_t)tq) << (BITS * s);
          }
          store_codes<BITS>(rec, k * LV + l, word);
        }
      } else {
        // Lloyd-Max: q = #{k : z > tau_k}
        constexpr int NT = (1 << BITS) - 1;
        float tau[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) tau[i] = 0.5f * (a.codebook[i] + a.codebook[i + 1]);
#pragma unroll
        for (int k = 0; k < kNC; ++k) {
          uint32_t word = 0;
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const float z = v[8 * k + s] * A;
            uint32_t c = 0;
#pragma unroll
            for (int i = 0; i < NT; ++i) c += (z > tau[i]) ? 1u : 0u;
            word |= c << (BITS * s);
          }
          store_codes<BITS>(rec, k * LV + l, word);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// DECODE
// ---------------------------------------------------------------------------
template <int ODT, int D, int BITS, int ROT, int QUANT>
__global__ void __launch_bounds__(64 * kWavesPerBlock) decode_kernel(const CodecArgs a) {
  using G = Geo<D>;
  constexpr int LV = G::LV, VPW = G::VPW;
  extern __shared__ float s_scratch[];
  __shared__ float s_mat[ROT == ROT_SO4 ? (D / 4) * 16 : 1];
  __shared__ float s_cb[kMaxCodebook];

  const int tid = threadIdx.x;
  if constexpr (ROT == ROT_SO4) {
    for (int b = tid; b < D / 4; b += blockDim.x) build_so4(&a.quat[8 * b], &s_mat[16 * b]);
  }
  if constexpr (QUANT == Q_LLOYD) {
    if (tid < (1 << BITS)) s_cb[tid] = a.codebook[tid];
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  int64_t block = blockIdx.x;
  if (a.xcd_remap) {
    const int64_t nb = gridDim.x;
    block = (block & 7) * (nb >> 3) + (block >> 3);
  }
  const int64_t item = block * kWavesPerBlock + wave;
  if (item >= (int64_t)a.n_tiles * a.n_row_chunks) return;

  const int tile = (int)(item % a.n_tiles);
  const int rc = (int)(item / a.n_tiles);
  const int q = lane / LV, l = lane % LV;
  const int64_t ncols = a.tokens * a.heads;
  const int64_t col = (int64_t)tile * VPW + q;
  const bool valid = col < ncols;
  const int64_t t = valid ? col / a.heads : 0;
  const int64_t h = valid ? col - t * a.heads : 0;
  const int64_t pos = a.pos_offset + t;
  const bool is_sink = valid && pos < a.n_sink;
  const bool work = valid && !is_sink;
  const int64_t r0 = (int64_t)rc * a.rows_per_item;
  const int64_t r1 = min(a.rows, r0 + a.rows_per_item);

  float* scratch = s_scratch + wave * VPW * G::STRIDE;
  int paddr[32];
  if (a.use_perm) {
#pragma unroll
    for (int k = 0; k < kNC; ++k)
#pragma unroll
      for (int s = 0; s < 8; ++s)
        paddr[8 * k + s] = q * G::STRIDE + (int)a.perm[(k * LV + l) * 8 + s];
  }
  const float norm_c = (ROT == ROT_FWHT) ? (float)(1.0 / __builtin_sqrt((double)D)) : 1.0f;
  const float sgn = (ROT == ROT_FWHT) ? lane_sign(l) : 1.0f;
  const int gb = a.group_log2;
  const int CB = (QUANT == Q_MINMAX) ? max(0, gb - 3 - G::LVB) : 0;
  const int64_t ngroups = (QUANT == Q_MINMAX) ? (D >> gb) : 0;

  for (int64_t r = r0; r < r1; ++r) {
    const int64_t vec = r * ncols + col;
    float v[32];
    if (is_sink) {
      const int64_t srow = (r * a.n_sink + pos) * a.heads + h;
#pragma unroll
      for (int k = 0; k < kNC; ++k) load_chunk<DT_F16>(a.sink, srow * D + (k * LV + l) * 8, v + 8 * k);
    }
    if (work) {
      const uint8_t* rec = a.codes + vec * (D * BITS / 8);
      if constexpr (QUANT == Q_MINMAX) {
#pragma unroll
        for (int k = 0; k < kNC; ++k) {
          const uint32_t word = load_codes<BITS>(rec, k * LV + l);
          const int64_t gi = ((int64_t)((k * LV + l) * 8)) >> gb;
          const float sc = f16_value(a.scale[vec * ngroups + gi]);
          const float z = f16_value(a.zero[vec * ngroups + gi]);
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const float qv = (float)((word >> (BITS * s)) & ((1u << BITS) - 1u));
            v[8 * k + s] = __builtin_fmaf(qv, sc, z);
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < kNC; ++k) {
          const uint32_t word = load_codes<BITS>(rec, k * LV + l);
#pragma unroll
          for (int s = 0; s < 8; ++s) v[8 * k + s] = s_cb[(word >> (BITS * s)) & ((1u << BITS) - 1u)];
        }
      }
      (void)CB;
      float outscale = 1.0f;
      if constexpr (ROT == ROT_FWHT) {
        fwht_lane<LV>(v, l);
        outscale = sgn * norm_c;
      } else if constexpr (ROT == ROT_SO4) {
        // inverse: M^T z (M orthogonal for unit quaternions)
#pragma unroll
        for (int k = 0; k < kNC; ++k)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int blk = (k * LV + l) * 2 + half;
            const float* m = &s_mat[16 * blk];
            float* u = v + 8 * k + 4 * half;
            const float u0 = u[0], u1 = u[1], u2 = u[2], u3 = u[3];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              u[i] = __builtin_fmaf(m[i], u0,
                     __builtin_fmaf(m[4 + i], u1, __builtin_fmaf(m[8 + i], u2, m[12 + i] * u3)));
          }
      }
      if constexpr (QUANT == Q_LLOYD) outscale *= a.norm[vec];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] *= outscale;
      if (a.use_perm) {
        // scatter: out[perm[j]] = v[j]
#pragma unroll
        for (int i = 0; i < 32; ++i) scratch[paddr[i]] = v[i];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int k = 0; k < kNC; ++k) {
          const float4* src = reinterpret_cast<const float4*>(scratch + q * G::STRIDE + (k * LV + l) * 8);
          const float4 p0 = src[0], p1 = src[1];
          v[8 * k] = p0.x; v[8 * k + 1] = p0.y; v[8 * k + 2] = p0.z; v[8 * k + 3] = p0.w;
          v[8 * k + 4] = p1.x; v[8 * k + 5] = p1.y; v[8 * k + 6] = p1.z; v[8 * k + 7] = p1.w;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
    if (valid) {
#pragma unroll
      for (int k = 0; k < kNC; ++k) store_chunk<ODT>(a.y, vec * D + (k * LV + l) * 8, v + 8 * k);
    }
  }
}

// ---------------------------------------------------------------------------
// launch dispatch
// ---------------------------------------------------------------------------
template <int D>
inline size_t scratch_bytes(const CodecArgs& a) {
  return a.use_perm ? (size_t)kWavesPerBlock * Geo<D>::VPW * Geo<D>::STRIDE * sizeof(float) : 0;
}

template <int D>
inline unsigned grid_blocks(const CodecArgs& a) {
  const int64_t items = (int64_t)a.n_tiles * a.n_row_chunks;
  return (unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock);
}

template <int DT, int D, int BITS, int ROT, int QUANT>
int launch_enc_t(const CodecArgs& a, hipStream_t s) {
  const unsigned nb = grid_blocks<D>(a);
  if (nb == 0) return 0;
  CodecArgs b = a;
  b.xcd_remap = (nb % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((encode_kernel<DT, D, BITS, ROT, QUANT>), dim3(nb), dim3(64 * kWavesPerBlock),
                     scratch_bytes<D>(a), s, b);
  return (int)hipGetLastError();
}

template <int ODT, int D, int BITS, int ROT, int QUANT>
int launch_dec_t(const CodecArgs& a, hipStream_t s) {
  const unsigned nb = grid_blocks<D>(a);
  if (nb == 0) return 0;
  CodecArgs b = a;
  b.xcd_remap = (nb % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((decode_kernel<ODT, D, BITS, ROT, QUANT>), dim3(nb), dim3(64 * kWavesPerBlock),
                     scratch_bytes<D>(a), s, b);
  return (int)hipGetLastError();
}

template <bool ENC, int DT, int D, int BITS, int ROT>
int pick_quant(int quant, const CodecArgs& a, hipStream_t s) {
  if (quant == Q_MINMAX)
    return ENC ? launch_enc_t<DT, D, BITS, ROT, Q_MINMAX>(a, s) : launch_dec_t<DT, D, BITS, ROT, Q_MINMAX>(a, s);
  return ENC ? launch_enc_t<DT, D, BITS, ROT, Q_LLOYD>(a, s) : launch_dec_t<DT, D, BITS, ROT, Q_LLOYD>(a, s);
}

template <bool ENC, int DT, int D, int BITS>
int pick_rot(int rot, int quant, const CodecArgs& a, hipStream_t s) {
  switch (rot) {
    case ROT_NONE: return pick_quant<ENC, DT, D, BITS, ROT_NONE>(quant, a, s);
    case ROT_FWHT: return pick_quant<ENC, DT, D, BITS, ROT_FWHT>(quant, a, s);
    default: return pick_quant<ENC, DT, D, BITS, ROT_SO4>(quant, a, s);
  }
}

template <bool ENC, int DT, int D>
int pick_bits(int bits, int rot, int quant, const CodecArgs& a, hipStream_t s) {
  switch (bits) {
    case 2: return pick_rot<ENC, DT, D, 2>(rot, quant, a, s);
    case 3: return pick_rot<ENC, DT, D, 3>(rot, quant, a, s);
    default: return pick_rot<ENC, DT, D, 4>(rot, quant, a, s);
  }
}

template <bool ENC, int DT>
int pick_dim(int d, int bits, int rot, int quant, const CodecArgs& a, hipStream_t s) {
  if (d == 128) return pick_bits<ENC, DT, 128>(bits, rot, quant, a, s);
  return pick_bits<ENC, DT, 256>(bits, rot, quant, a, s);
}

}  // namespace

// One translation unit per (direction, dtype) when KVQ_UNIT is 0..5, so the
// 216 kernel instances build in parallel; without KVQ_UNIT every launcher is
// defined here.
#ifndef KVQ_UNIT
#define KVQ_UNIT -1
#endif

#define KVQ_DEFINE_LAUNCH(NAME, ENC, DT)                                                      \
  int NAME(int head_dim, int bits, int rot, int quant, const CodecArgs& a, void* stream) {    \
    return pick_dim<ENC, DT>(head_dim, bits, rot, quant, a, reinterpret_cast<hipStream_t>(stream)); \
  }

#if KVQ_UNIT == 0 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_encode_f16, true, DT_F16)
const char* device_error_string(int err) { return hipGetErrorString((hipError_t)err); }
#endif
#if KVQ_UNIT == 1 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_encode_bf16, true, DT_BF16)
#endif
#if KVQ_UNIT == 2 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_encode_f32, true, DT_F32)
#endif
#if KVQ_UNIT == 3 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_decode_f16, false, DT_F16)
#endif
#if KVQ_UNIT == 4 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_decode_bf16, false, DT_BF16)
#endif
#if KVQ_UNIT == 5 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_decode_f32, false, DT_F32)
#endif

}  // namespace kvq
