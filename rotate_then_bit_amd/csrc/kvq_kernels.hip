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

#include <algorithm>
#include <atomic>

#include "kvq_internal.h"

namespace kvq {
namespace {

enum { DT_F16 = 0, DT_BF16 = 1, DT_F32 = 2 };
enum { ROT_NONE = 0, ROT_FWHT = 1, ROT_SO4 = 2 };
enum { Q_MINMAX = 0, Q_LLOYD = 1 };

constexpr int kNC = 4;  // 8-element chunks per lane (32 elements per lane)

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct Geo {
  static constexpr int LV = D / 32;                 // lanes per vector
  static constexpr int LVB = (LV == 4) ? 2 : 3;      // log2(LV)
  static constexpr int VPW = 64 / LV;                // vectors per wave
  static constexpr int STRIDE = D + 4;               // floats per vector in the perm scratch
};

// Per-wave LDS scratch: VPW vectors of STRIDE floats for the permutation, which in the
// encoder first holds the RoPE cos/sin table of the wave's current tile (at most VPW
// tokens x D/2 pairs of float2 = VPW * D * 4 bytes, less than the permutation's need).
template <int D>
constexpr int scratch_wave_bytes() {
  return Geo<D>::VPW * Geo<D>::STRIDE * 4;
}
static_assert(Geo<128>::VPW * 128 * 4 <= scratch_wave_bytes<128>(), "trig table fits");
static_assert(Geo<256>::VPW * 256 * 4 <= scratch_wave_bytes<256>(), "trig table fits");

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
template <int LV, bool FIRST_DONE = false>
__device__ __forceinline__ void fwht_lane(float* v, int l) {
  // slot bits (s = 0..7 within each chunk); the bit-0 stage may already have been
  // applied while widening 16-bit input pairs
#pragma unroll
  for (int hb = FIRST_DONE ? 2 : 1; hb < 8; hb <<= 1) {
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
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
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

// 8 elements to ``p``.  Plain stores: with this kernel's store pattern (each wave64
// store covers a 64-byte run in each of 16 vector records) non-temporal stores were
// measured at about half the bandwidth of ordinary ones on MI355X.
template <int DT>
__device__ __forceinline__ void store_chunk_at(char* p, const float* v) {
  if constexpr (DT == DT_F32) {
    u32x4_t a, b;
    a.x = __float_as_uint(v[0]); a.y = __float_as_uint(v[1]); a.z = __float_as_uint(v[2]); a.w = __float_as_uint(v[3]);
    b.x = __float_as_uint(v[4]); b.y = __float_as_uint(v[5]); b.z = __float_as_uint(v[6]); b.w = __float_as_uint(v[7]);
    reinterpret_cast<u32x4_t*>(p)[0] = a;
    reinterpret_cast<u32x4_t*>(p)[1] = b;
  } else {
    u32x4_t w;
    if constexpr (DT == DT_BF16) {
      w.x = pack_bf16x2(v[0], v[1]); w.y = pack_bf16x2(v[2], v[3]);
      w.z = pack_bf16x2(v[4], v[5]); w.w = pack_bf16x2(v[6], v[7]);
    } else {
      w.x = f16_bits(v[0]) | (f16_bits(v[1]) << 16); w.y = f16_bits(v[2]) | (f16_bits(v[3]) << 16);
      w.z = f16_bits(v[4]) | (f16_bits(v[5]) << 16); w.w = f16_bits(v[6]) | (f16_bits(v[7]) << 16);
    }
    *reinterpret_cast<u32x4_t*>(p) = w;
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

// Same layout, with ``p`` already pointing at chunk ``chunk``'s first byte.
template <int BITS>
__device__ __forceinline__ void store_codes_at(uint8_t* p, int chunk, uint32_t word) {
  if constexpr (BITS == 2) {
    *reinterpret_cast<uint16_t*>(p) = (uint16_t)word;
  } else if constexpr (BITS == 4) {
    *reinterpret_cast<uint32_t*>(p) = word;
  } else {
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
__device__ __forceinline__ uint32_t load_codes_at(const uint8_t* p, int chunk) {
  if constexpr (BITS == 2) {
    return *reinterpret_cast<const uint16_t*>(p);
  } else if constexpr (BITS == 4) {
    return *reinterpret_cast<const uint32_t*>(p);
  } else {
    if ((chunk & 1) == 0)
      return (uint32_t)*reinterpret_cast<const uint16_t*>(p) | ((uint32_t)p[2] << 16);
    return (uint32_t)p[0] | ((uint32_t)*reinterpret_cast<const uint16_t*>(p + 1) << 8);
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
// per-lane row storage and the work item shared by both kernels
// ---------------------------------------------------------------------------
// Raw input of one lane for one row: 4 chunks of 8 elements (16 bytes per chunk
// for 16-bit types, 32 bytes for float).
template <int DT>
struct RawRow {
  static constexpr int NW = (DT == DT_F32) ? 8 : 4;
  u32x4_t w[NW];
};

// Loads of one row: ``rowbase`` is wave-uniform, ``loff`` the lane's byte offset from it
// (32-bit), so the loads use a scalar base with a vector offset.
template <int DT, int LV>
__device__ __forceinline__ void load_row(RawRow<DT>& raw, const char* rowbase, uint32_t loff) {
  constexpr int ES = (DT == DT_F32) ? 4 : 2;
  const char* b = rowbase + loff;
#pragma unroll
  for (int k = 0; k < kNC; ++k) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(b + k * LV * 8 * ES);
    if constexpr (DT == DT_F32) {
      raw.w[2 * k] = __builtin_nontemporal_load(p);
      raw.w[2 * k + 1] = __builtin_nontemporal_load(p + 1);
    } else {
      raw.w[k] = __builtin_nontemporal_load(p);
    }
  }
}

template <int DT>
__device__ __forceinline__ void widen_row(const RawRow<DT>& raw, float* v) {
#pragma unroll
  for (int k = 0; k < kNC; ++k) {
    if constexpr (DT == DT_F32) {
      const u32x4_t a = raw.w[2 * k], b = raw.w[2 * k + 1];
      v[8 * k + 0] = __uint_as_float(a.x); v[8 * k + 1] = __uint_as_float(a.y);
      v[8 * k + 2] = __uint_as_float(a.z); v[8 * k + 3] = __uint_as_float(a.w);
      v[8 * k + 4] = __uint_as_float(b.x); v[8 * k + 5] = __uint_as_float(b.y);
      v[8 * k + 6] = __uint_as_float(b.z); v[8 * k + 7] = __uint_as_float(b.w);
    } else {
      const uint32_t ws[4] = {raw.w[k].x, raw.w[k].y, raw.w[k].z, raw.w[k].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (DT == DT_BF16) {
          v[8 * k + 2 * i] = __uint_as_float(ws[i] << 16);
          v[8 * k + 2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
        } else {
          v[8 * k + 2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws[i] & 0xffffu));
          v[8 * k + 2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws[i] >> 16));
        }
      }
    }
  }
}

// Widen a 16-bit row and apply the first Walsh-Hadamard stage (channel pairs 2i, 2i+1,
// which share a dword) in one step: dot2(pair, (1, 1)) and dot2(pair, (1, -1)) form
// x0 + x1 and x0 - x1 in float with a single rounding, like the float adds they replace.
template <int DT>
__device__ __forceinline__ void widen_row_butterfly(const RawRow<DT>& raw, float* v) {
  static_assert(DT != DT_F32, "16-bit inputs only");
#pragma unroll
  for (int k = 0; k < kNC; ++k) {
    const uint32_t ws[4] = {raw.w[k].x, raw.w[k].y, raw.w[k].z, raw.w[k].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == DT_BF16) {
        const bf16x2_t pr = __builtin_bit_cast(bf16x2_t, ws[i]);
        const bf16x2_t pp = {(__bf16)1.0f, (__bf16)1.0f};
        const bf16x2_t pm = {(__bf16)1.0f, (__bf16)-1.0f};
        v[8 * k + 2 * i] = __builtin_amdgcn_fdot2_f32_bf16(pr, pp, 0.0f, false);
        v[8 * k + 2 * i + 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, pm, 0.0f, false);
      } else {
        const f16x2_t pr = __builtin_bit_cast(f16x2_t, ws[i]);
        const f16x2_t pp = {(_Float16)1.0f, (_Float16)1.0f};
        const f16x2_t pm = {(_Float16)1.0f, (_Float16)-1.0f};
        v[8 * k + 2 * i] = __builtin_amdgcn_fdot2(pr, pp, 0.0f, false);
        v[8 * k + 2 * i + 1] = __builtin_amdgcn_fdot2(pr, pm, 0.0f, false);
      }
    }
  }
}

// A wave's position in the row-major item sequence: row r, tile (VPW consecutive
// (token, head) columns starting at col0 = tile * VPW = t0 * heads + h0).  All fields
// are wave-uniform; the step from one of the wave's items to the next is a fixed
// (rows, tiles) increment, so no division is needed after the first item.
struct Cursor {
  int64_t r, tile, t0, h0;
};

template <int VPW>
__device__ __forceinline__ Cursor first_cursor(const CodecArgs& a, int64_t wid) {
  Cursor c;
  c.r = wid / a.n_tiles;
  c.tile = wid - c.r * a.n_tiles;
  const int64_t col0 = c.tile * VPW;
  c.t0 = col0 / a.heads;
  c.h0 = col0 - c.t0 * a.heads;
  return c;
}

__device__ __forceinline__ void advance(const CodecArgs& a, Cursor& c) {
  c.tile += a.step_tiles;
  c.r += a.step_rows;
  c.h0 += a.step_head;
  c.t0 += a.step_tok;
  if (c.h0 >= a.heads) { c.h0 -= a.heads; c.t0 += 1; }
  if (c.tile >= a.n_tiles) {
    c.tile -= a.n_tiles;
    c.r += 1;
    c.h0 -= a.wrap_head;
    c.t0 -= a.wrap_tok;
    if (c.h0 < 0) { c.h0 += a.heads; c.t0 -= 1; }
  }
}

// Token offset from t0 and head of the lane's vector q in the tile: (h0 + q) / heads by
// a multiply-high with ceil(2^32 / heads), exact for h0 + q < heads + 64 <= 2^16 + 64.
__device__ __forceinline__ void lane_token_head(const CodecArgs& a, const Cursor& c, int q, int& dtok, int& head) {
  const uint32_t hq = (uint32_t)(c.h0 + q);
  const uint32_t d = (a.heads == 1) ? hq : __umulhi(hq, a.heads_magic);
  dtok = (int)d;
  head = (int)(hq - d * (uint32_t)a.heads);
}

// Permutation gather offsets (bytes) for lane-in-vector l and slot i = 8k + s:
// perm[(k*LV + l)*8 + s] * 4, staged in LDS once per block.
template <int D>
__device__ __forceinline__ void stage_perm_offsets(const CodecArgs& a, int* s_poff) {
  constexpr int LV = Geo<D>::LV;
  for (int i = threadIdx.x; i < LV * 32; i += blockDim.x) {
    const int l = i / 32, slot = i % 32, k = slot / 8, s = slot % 8;
    s_poff[i] = 4 * (int)a.perm[(k * LV + l) * 8 + s];
  }
}

// ---------------------------------------------------------------------------
// ENCODE
// ---------------------------------------------------------------------------
// RT / PT: RoPE / permutation off (0), on (1) or read from the arguments (-1).
// GBT: log2 of the min-max group size, or -1 to read it from the arguments.  The hot
// configurations get compile-time values; the rest share run-time variants.
template <int DT, int D, int BITS, int ROT, int QUANT, int RT, int PT, int GBT>
__global__ void __launch_bounds__(64 * kWavesPerBlock) encode_kernel(const CodecArgs a) {
  using G = Geo<D>;
  constexpr int LV = G::LV, VPW = G::VPW;
  constexpr bool ROPE_ANY = RT != 0, PERM_ANY = PT != 0;
  const bool ROPE = (RT < 0) ? (a.rope != 0) : (RT == 1);
  const bool PERM = (PT < 0) ? (a.use_perm != 0) : (PT == 1);
  extern __shared__ float s_scratch[];
  __shared__ double s_theta[ROPE_ANY ? D / 2 : 1];
  __shared__ float s_mat[ROT == ROT_SO4 ? (D / 4) * 16 : 1];
  __shared__ int s_poff[PERM_ANY ? LV * 32 : 1];

  const int tid = threadIdx.x;
  if constexpr (ROPE_ANY) {
    if (ROPE)
      for (int i = tid; i < D / 2; i += blockDim.x)
        s_theta[i] = exp2(-(2.0 * (double)i / (double)D) * a.rope_log2_base);
  }
  if constexpr (ROT == ROT_SO4) {
    for (int b = tid; b < D / 4; b += blockDim.x) build_so4(&a.quat[8 * b], &s_mat[16 * b]);
  }
  if constexpr (PERM_ANY) {
    if (PERM) stage_perm_offsets<D>(a, s_poff);
  }
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t wid = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (wid >= a.n_items) return;  // wave-uniform; no barrier follows

  const int q = lane / LV, l = lane % LV;
  const int64_t ncols = a.tokens * a.heads;
  constexpr int ES = (DT == DT_F32) ? 4 : 2;
  constexpr int CBYTES = D * BITS / 8;  // code bytes per vector
  const uint32_t clane = (uint32_t)(q * CBYTES + l * BITS);

  // per-wave LDS: the permutation scratch, which also holds the RoPE cos/sin table of
  // the current item until the rotation has consumed it
  char* wscratch = reinterpret_cast<char*>(s_scratch) + wave * scratch_wave_bytes<D>();
  char* vscratch = wscratch + q * G::STRIDE * 4;
  const int* poff = s_poff + l * 32;

  const float norm_c = (ROT == ROT_FWHT) ? (float)(1.0 / __builtin_sqrt((double)D)) : 1.0f;
  const float sgn = (ROT == ROT_FWHT) ? lane_sign(l) : 1.0f;
  const float A = sgn * norm_c;  // true rotated coefficient = A * (value held by this lane)
  const int gb = (GBT > 0) ? GBT : a.group_log2;
  const int LB = (QUANT == Q_MINMAX) ? min(G::LVB, gb - 3) : 0;     // lane bits inside a group
  const int CB = (QUANT == Q_MINMAX) ? max(0, gb - 3 - G::LVB) : 0; // chunk bits inside a group
  const int64_t ngroups = (QUANT == Q_MINMAX) ? (D >> gb) : 0;

  // 16-bit input straight into the transform: widen and first butterfly stage fused
  constexpr bool FUSED = (DT != DT_F32) && RT == 0 && PT == 0 && (QUANT == Q_MINMAX) && (ROT == ROT_FWHT);

  // input address of the lane's vector for an item: wave-uniform base, 32-bit lane offset
  auto input_of = [&](const Cursor& c, const char*& base, uint32_t& loff, bool& valid) {
    int dtok, head;
    lane_token_head(a, c, q, dtok, head);
    valid = c.tile * VPW + q < ncols;
    base = reinterpret_cast<const char*>(a.x) + (c.r * a.sr + c.t0 * a.st) * ES;
    loff = (uint32_t)(((int64_t)dtok * a.st + (int64_t)head * a.sh + (int64_t)l * 8) * ES);
  };

  auto process = [&](const RawRow<DT>& raw, const Cursor& c) {
    const int64_t r = c.r;
    const int64_t col0 = c.tile * VPW;
    int dtok, h;
    lane_token_head(a, c, q, dtok, h);
    const int64_t col = col0 + q;
    const bool valid = col < ncols;
    const int64_t pos = a.pos_offset + c.t0 + dtok;
    const bool is_sink = valid && pos < a.n_sink;
    const bool work = valid && !is_sink;
    const int64_t vec = r * ncols + col;  // index into the packed planes
    const int64_t vec0 = r * ncols + col0;  // wave-uniform
    uint8_t* rec = a.codes + vec0 * CBYTES + clane;  // chunk c of this lane at rec + (c - l) * BITS
    float v[32];
    if constexpr (FUSED) {
      if (is_sink) widen_row<DT>(raw, v);  // sinks store the unrotated values
      else widen_row_butterfly<DT>(raw, v);
    } else {
      widen_row<DT>(raw, v);
    }
    if (ROPE_ANY && ROPE) {
      // cos/sin of (position, pair) for the tokens of this tile, computed once per item
      // by the whole wave into LDS (about 2 angles per lane when heads = 8)
      const int ntok = (int)((c.h0 + VPW - 1) / a.heads) + 1;
      float2* trig = reinterpret_cast<float2*>(wscratch);
      for (int m = lane; m < ntok * (D / 2); m += 64) {
        const int tok = m / (D / 2), i = m % (D / 2);
        float cs, sn;
        rope_cos_sin(a.pos_offset + c.t0 + tok, s_theta[i], &cs, &sn);
        trig[m] = make_float2(cs, sn);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (valid) {
        const float4* tl = reinterpret_cast<const float4*>(trig + dtok * (D / 2));
#pragma unroll
        for (int k = 0; k < kNC; ++k) {
          const float4 p01 = tl[(k * LV + l) * 2], p23 = tl[(k * LV + l) * 2 + 1];
          const float cc[4] = {p01.x, p01.z, p23.x, p23.z};
          const float ss[4] = {p01.y, p01.w, p23.y, p23.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x0 = v[8 * k + 2 * j], x1 = v[8 * k + 2 * j + 1];
            v[8 * k + 2 * j] = __builtin_fmaf(x0, cc[j], -x1 * ss[j]);
            v[8 * k + 2 * j + 1] = __builtin_fmaf(x0, ss[j], x1 * cc[j]);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (!valid) return;
    if (is_sink) {
      const int64_t srow = (r * a.n_sink + pos) * a.heads + h;
#pragma unroll
      for (int k = 0; k < kNC; ++k) store_chunk<DT_F16>(a.sink, srow * D + (k * LV + l) * 8, v + 8 * k);
#pragma unroll
      for (int k = 0; k < kNC; ++k) store_codes_at<BITS>(rec + k * LV * BITS, k * LV + l, 0u);
      if constexpr (QUANT == Q_MINMAX) {
        for (int g = l; g < ngroups; g += LV) {
          a.scale[vec * ngroups + g] = 0;
          a.zero[vec * ngroups + g] = 0;
        }
      } else {
        if (l == 0) a.norm[vec] = 0.0f;
      }
    }
    if (!work) return;
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
    if (PERM_ANY && PERM) {
      // natural order in, gathered order out: u'[j] = u[perm[j]] (one wave, in-order LDS)
#pragma unroll
      for (int k = 0; k < kNC; ++k) {
        float4* dst = reinterpret_cast<float4*>(vscratch + 32 * (k * LV + l));
        dst[0] = make_float4(v[8 * k], v[8 * k + 1], v[8 * k + 2], v[8 * k + 3]);
        dst[1] = make_float4(v[8 * k + 4], v[8 * k + 5], v[8 * k + 6], v[8 * k + 7]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        const int4 o = *reinterpret_cast<const int4*>(poff + i);
        v[i] = *reinterpret_cast<const float*>(vscratch + o.x);
        v[i + 1] = *reinterpret_cast<const float*>(vscratch + o.y);
        v[i + 2] = *reinterpret_cast<const float*>(vscratch + o.z);
        v[i + 3] = *reinterpret_cast<const float*>(vscratch + o.w);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if constexpr (ROT == ROT_FWHT) {
      fwht_lane<LV, FUSED>(v, l);
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
    if constexpr (QUANT == Q_MINMAX) {
      // min/max of the lane's values of each group (a group covers 1, 2 or 4 of the
      // lane's chunks); the true coefficients are A * v, so for A < 0 min and max swap
      float cmn[kNC], cmx[kNC];
      auto mm8 = [&](int k, float& lo, float& hi) {
        const float* c = v + 8 * k;
        lo = fminf(fminf(fminf(c[0], c[1]), fminf(c[2], c[3])), fminf(fminf(c[4], c[5]), fminf(c[6], c[7])));
        hi = fmaxf(fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3])), fmaxf(fmaxf(c[4], c[5]), fmaxf(c[6], c[7])));
      };
      auto orient = [&](float lo, float hi, float& mn, float& mx) {
        mn = (A > 0.0f) ? lo * A : hi * A;
        mx = (A > 0.0f) ? hi * A : lo * A;
      };
      if (CB == 2) {
        float lo, hi, lo1, hi1, lo2, hi2, lo3, hi3;
        mm8(0, lo, hi); mm8(1, lo1, hi1); mm8(2, lo2, hi2); mm8(3, lo3, hi3);
        lo = fminf(fminf(lo, lo1), fminf(lo2, lo3));
        hi = fmaxf(fmaxf(hi, hi1), fmaxf(hi2, hi3));
        orient(lo, hi, cmn[0], cmx[0]);
      } else if (CB == 1) {
        float lo, hi, lo1, hi1;
        mm8(0, lo, hi); mm8(1, lo1, hi1);
        orient(fminf(lo, lo1), fmaxf(hi, hi1), cmn[0], cmx[0]);
        mm8(2, lo, hi); mm8(3, lo1, hi1);
        orient(fminf(lo, lo1), fmaxf(hi, hi1), cmn[2], cmx[2]);
      } else {
#pragma unroll
        for (int k = 0; k < kNC; ++k) {
          float lo, hi;
          mm8(k, lo, hi);
          orient(lo, hi, cmn[k], cmx[k]);
        }
      }
      // per-group zero/scale: reduce over the group's lanes, round to fp16
      // (zero down, scale up), store from the group's first lane
      auto group = [&](float mn, float mx, int k, float& zo, float& so, float& io) {
        if (LB >= 1) { mn = min_x1(mn); mx = max_x1(mx); }
        if (LB >= 2) { mn = min_x2(mn); mx = max_x2(mx); }
        if (LB >= 3) { mn = fminf(mn, swz_x4(mn)); mx = fmaxf(mx, swz_x4(mx)); }
        // "+ 0.0f" turns a -0 (all-zero group, negated lanes) into +0
        const uint32_t zb = f16_round_down(mn + 0.0f);
        const float z = f16_value(zb);
        // (max - zero) / (2^b - 1) to within an ulp, then rounded up to fp16
        constexpr float kInvLevels = 1.0f / (float)((1 << BITS) - 1);
        const uint32_t sb = f16_round_up((mx - z) * kInvLevels + 0.0f);
        const float sc = f16_value(sb);
        if ((l & ((1 << LB) - 1)) == 0) {
          const int64_t gi = ((int64_t)((k * LV + l) * 8)) >> gb;
          a.scale[vec * ngroups + gi] = (uint16_t)sb;
          a.zero[vec * ngroups + gi] = (uint16_t)zb;
        }
        zo = z;
        so = sc;
        io = (sc > 0.0f) ? __builtin_amdgcn_rcpf(sc) : 0.0f;
      };
      float zf[kNC], inv[kNC], scf[kNC];
      group(cmn[0], cmx[0], 0, zf[0], scf[0], inv[0]);
      if (CB == 0) {
        group(cmn[1], cmx[1], 1, zf[1], scf[1], inv[1]);
        group(cmn[2], cmx[2], 2, zf[2], scf[2], inv[2]);
        group(cmn[3], cmx[3], 3, zf[3], scf[3], inv[3]);
      } else if (CB == 1) {
        group(cmn[2], cmx[2], 2, zf[2], scf[2], inv[2]);
        zf[1] = zf[0]; inv[1] = inv[0]; scf[1] = scf[0];
        zf[3] = zf[2]; inv[3] = inv[2]; scf[3] = scf[2];
      } else {
        zf[1] = zf[2] = zf[3] = zf[0];
        inv[1] = inv[2] = inv[3] = inv[0];
        scf[1] = scf[2] = scf[3] = scf[0];
      }
      // q = rint((A v - zero) / scale), nearest-even: adding 1.5 * 2^23 inside the fma
      // rounds the exact product to an integer, which then sits in the low mantissa bits
      // (bit pattern 0x4B400000 + q, since -eps <= t <= 2^b - 1 + eps).  The codes are
      // accumulated as (pattern << BITS*s) sums and the constant part subtracted once.
      constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
      constexpr uint32_t kMagicSum = [] {
        uint32_t c = 0;
        for (int s = 0; s < 8; ++s) c += 0x4B400000u << (BITS * s);
        return c;
      }();
#pragma unroll
      for (int k = 0; k < kNC; ++k) {
        const float z = zf[k], iv = inv[k], sc = scf[k];
        uint32_t word = 0;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const float d = __builtin_fmaf(v[8 * k + s], A, -z);
          float tq;
          if constexpr (ROT == ROT_NONE) {
            // unrotated fp16/bf16 data sit on the same grid as zero/scale, so exact
            // half-way quotients are common: one residual step makes d/scale correctly
            // rounded before the integer rounding
            const float t0 = d * iv;
            const float t1 = __builtin_fmaf(__builtin_fmaf(-t0, sc, d), iv, t0);
            tq = (sc > 0.0f ? t1 : 0.0f) + kMagic;
          } else {
            (void)sc;
            tq = __builtin_fmaf(d, iv, kMagic);
          }
          word += __float_as_uint(tq) << (BITS * s);
        }
        store_codes_at<BITS>(rec + k * LV * BITS, k * LV + l, word - kMagicSum);
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
        store_codes_at<BITS>(rec + k * LV * BITS, k * LV + l, word);
      }
    }
  };

  // persistent loop over the wave's items with the next item's loads in flight
  Cursor ca = first_cursor<VPW>(a, wid);
  RawRow<DT> ra, rb;
  const char* xb;
  uint32_t xl;
  bool ok;
  input_of(ca, xb, xl, ok);
  if (ok) load_row<DT, LV>(ra, xb, xl);
  for (int64_t it = wid; it < a.n_items; it += 2 * a.n_waves) {
    Cursor cb = ca;
    advance(a, cb);
    const bool has_b = it + a.n_waves < a.n_items;
    if (has_b) {
      input_of(cb, xb, xl, ok);
      if (ok) load_row<DT, LV>(rb, xb, xl);
    }
    process(ra, ca);
    if (!has_b) break;
    ca = cb;
    advance(a, ca);
    if (it + 2 * a.n_waves < a.n_items) {
      input_of(ca, xb, xl, ok);
      if (ok) load_row<DT, LV>(ra, xb, xl);
    }
    process(rb, cb);
  }
}

// ---------------------------------------------------------------------------
// DECODE
// ---------------------------------------------------------------------------
// PT: permutation off (0), on (1) or read from the arguments (-1).
template <int ODT, int D, int BITS, int ROT, int QUANT, int PT>
__global__ void __launch_bounds__(64 * kWavesPerBlock) decode_kernel(const CodecArgs a) {
  using G = Geo<D>;
  constexpr int LV = G::LV, VPW = G::VPW;
  constexpr bool PERM_ANY = PT != 0;
  const bool PERM = (PT < 0) ? (a.use_perm != 0) : (PT == 1);
  extern __shared__ float s_scratch[];
  __shared__ float s_mat[ROT == ROT_SO4 ? (D / 4) * 16 : 1];
  __shared__ float s_cb[kMaxCodebook];
  __shared__ int s_poff[PERM_ANY ? LV * 32 : 1];

  const int tid = threadIdx.x;
  if constexpr (ROT == ROT_SO4) {
    for (int b = tid; b < D / 4; b += blockDim.x) build_so4(&a.quat[8 * b], &s_mat[16 * b]);
  }
  if constexpr (QUANT == Q_LLOYD) {
    if (tid < (1 << BITS)) s_cb[tid] = a.codebook[tid];
  }
  if constexpr (PERM_ANY) {
    if (PERM) stage_perm_offsets<D>(a, s_poff);
  }
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t wid = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (wid >= a.n_items) return;  // wave-uniform; no barrier follows

  const int q = lane / LV, l = lane % LV;
  const int64_t ncols = a.tokens * a.heads;

  char* vscratch = reinterpret_cast<char*>(s_scratch) + wave * scratch_wave_bytes<D>() + q * G::STRIDE * 4;
  const int* poff = s_poff + l * 32;
  const float norm_c = (ROT == ROT_FWHT) ? (float)(1.0 / __builtin_sqrt((double)D)) : 1.0f;
  const float sgn = (ROT == ROT_FWHT) ? lane_sign(l) : 1.0f;
  const int gb = a.group_log2;
  const int64_t ngroups = (QUANT == Q_MINMAX) ? (D >> gb) : 0;

  // packed inputs of one vector for this lane: code words of its 4 chunks, plus the
  // scale/zero of each chunk's group (min-max) or rho (Lloyd-Max)
  struct Packed {
    uint32_t word[kNC];
    uint32_t sz[kNC];  // scale | zero << 16
    float rho;
  };
  constexpr int CBYTES = D * BITS / 8;
  const uint32_t clane = (uint32_t)(q * CBYTES + l * BITS);
  // a lane's vector of an item: validity, sink test and (for sinks) the sink record
  auto lane_state = [&](const Cursor& c, bool& valid, bool& is_sink, int64_t& srow) {
    int dtok, h;
    lane_token_head(a, c, q, dtok, h);
    valid = c.tile * VPW + q < ncols;
    const int64_t pos = a.pos_offset + c.t0 + dtok;
    is_sink = valid && pos < a.n_sink;
    srow = (c.r * a.n_sink + pos) * a.heads + h;
  };
  auto load_packed = [&](Packed& pk, const Cursor& c) {
    const int64_t vec0 = c.r * ncols + c.tile * VPW;  // wave-uniform
    const uint8_t* rec = a.codes + vec0 * CBYTES + clane;
#pragma unroll
    for (int k = 0; k < kNC; ++k) pk.word[k] = load_codes_at<BITS>(rec + k * LV * BITS, k * LV + l);
    if constexpr (QUANT == Q_MINMAX) {
      const uint16_t* sp = a.scale + vec0 * ngroups + q * ngroups;
      const uint16_t* zp = a.zero + vec0 * ngroups + q * ngroups;
#pragma unroll
      for (int k = 0; k < kNC; ++k) {
        const int gi = ((k * LV + l) * 8) >> gb;
        pk.sz[k] = (uint32_t)sp[gi] | ((uint32_t)zp[gi] << 16);
      }
    } else {
      pk.rho = a.norm[vec0 + q];
    }
  };

  auto process = [&](const Packed& pk, const Cursor& c) {
    bool valid, is_sink;
    int64_t srow;
    lane_state(c, valid, is_sink, srow);
    if (!valid) return;
    float v[32];
    if (is_sink) {
#pragma unroll
      for (int k = 0; k < kNC; ++k) load_chunk<DT_F16>(a.sink, srow * D + (k * LV + l) * 8, v + 8 * k);
    } else {
      if constexpr (QUANT == Q_MINMAX) {
#pragma unroll
        for (int k = 0; k < kNC; ++k) {
          const float sc = f16_value(pk.sz[k] & 0xffffu);
          const float z = f16_value(pk.sz[k] >> 16);
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const float qv = (float)((pk.word[k] >> (BITS * s)) & ((1u << BITS) - 1u));
            v[8 * k + s] = __builtin_fmaf(qv, sc, z);
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < kNC; ++k)
#pragma unroll
          for (int s = 0; s < 8; ++s) v[8 * k + s] = s_cb[(pk.word[k] >> (BITS * s)) & ((1u << BITS) - 1u)];
      }
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
      if constexpr (QUANT == Q_LLOYD) outscale *= pk.rho;
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] *= outscale;
      if (PERM_ANY && PERM) {
        // scatter: out[perm[j]] = v[j], then read back in natural order
#pragma unroll
        for (int i = 0; i < 32; i += 4) {
          const int4 o = *reinterpret_cast<const int4*>(poff + i);
          *reinterpret_cast<float*>(vscratch + o.x) = v[i];
          *reinterpret_cast<float*>(vscratch + o.y) = v[i + 1];
          *reinterpret_cast<float*>(vscratch + o.z) = v[i + 2];
          *reinterpret_cast<float*>(vscratch + o.w) = v[i + 3];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int k = 0; k < kNC; ++k) {
          const float4* src = reinterpret_cast<const float4*>(vscratch + 32 * (k * LV + l));
          const float4 p0 = src[0], p1 = src[1];
          v[8 * k] = p0.x; v[8 * k + 1] = p0.y; v[8 * k + 2] = p0.z; v[8 * k + 3] = p0.w;
          v[8 * k + 4] = p1.x; v[8 * k + 5] = p1.y; v[8 * k + 6] = p1.z; v[8 * k + 7] = p1.w;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
    constexpr int OES = (ODT == DT_F32) ? 4 : 2;
    char* yrow = reinterpret_cast<char*>(a.y) + (c.r * ncols + c.tile * VPW) * D * OES;  // wave-uniform
    const uint32_t ylane = (uint32_t)((q * D + l * 8) * OES);
#pragma unroll
    for (int k = 0; k < kNC; ++k) store_chunk_at<ODT>(yrow + ylane + k * LV * 8 * OES, v + 8 * k);
  };

  // persistent loop over the wave's items with the next item's loads in flight
  auto fetch = [&](Packed& pk, const Cursor& c) {
    bool valid, is_sink;
    int64_t srow;
    lane_state(c, valid, is_sink, srow);
    if (valid && !is_sink) load_packed(pk, c);
  };
  Cursor ca = first_cursor<VPW>(a, wid);
  Packed pa, pb;
  fetch(pa, ca);
  for (int64_t it = wid; it < a.n_items; it += 2 * a.n_waves) {
    Cursor cb = ca;
    advance(a, cb);
    const bool has_b = it + a.n_waves < a.n_items;
    if (has_b) fetch(pb, cb);
    process(pa, ca);
    if (!has_b) break;
    ca = cb;
    advance(a, ca);
    if (it + 2 * a.n_waves < a.n_items) fetch(pa, ca);
    process(pb, cb);
  }
}

// ---------------------------------------------------------------------------
// launch dispatch
// ---------------------------------------------------------------------------
// Grid of a persistent launch: as many blocks as can be resident at once (occupancy
// of this kernel instance x compute units), but no more than there are items.  The
// cursor step constants follow from the wave count.
// Grid of a persistent launch: as many blocks as can be resident at once (occupancy
// of the kernel instance x compute units), but no more than there are items.  The
// cursor step constants follow from the wave count.  ``per_cu`` caches the occupancy
// of the instance (a property of the kernel and the gfx950 target, 0 = not yet known).
template <int D>
int plan_grid(const void* kernel, size_t lds, int& per_cu, CodecArgs& b, unsigned& nb) {
  constexpr int VPW = Geo<D>::VPW;
  static thread_local int cached_dev = -1, cu = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev != cached_dev) {
    e = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return (int)e;
    cached_dev = dev;
  }
  if (per_cu <= 0) {
    int n = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 64 * kWavesPerBlock, lds);
    if (e != hipSuccess) return (int)e;
    per_cu = n < 1 ? 1 : n;
  }
  const int64_t need = (b.n_items + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t blocks = std::min<int64_t>(need, (int64_t)per_cu * cu);
  nb = (unsigned)blocks;
  b.n_waves = blocks * kWavesPerBlock;
  b.step_rows = b.n_waves / b.n_tiles;
  b.step_tiles = b.n_waves % b.n_tiles;
  b.step_tok = b.step_tiles * VPW / b.heads;
  b.step_head = b.step_tiles * VPW % b.heads;
  b.wrap_tok = b.n_tiles * VPW / b.heads;
  b.wrap_head = b.n_tiles * VPW % b.heads;
  b.heads_magic = (b.heads >= 2) ? (uint32_t)(((1ull << 32) + (uint64_t)b.heads - 1) / (uint64_t)b.heads) : 0u;
  return 0;
}

template <int D>
inline size_t scratch_bytes(bool needed) {
  return needed ? (size_t)kWavesPerBlock * scratch_wave_bytes<D>() : 0;
}

template <int DT, int D, int BITS, int ROT, int QUANT, int RT, int PT, int GBT>
int launch_enc_t(const CodecArgs& a, hipStream_t s) {
  if (a.n_items == 0) return 0;
  const void* k = reinterpret_cast<const void*>(&encode_kernel<DT, D, BITS, ROT, QUANT, RT, PT, GBT>);
  const size_t lds = scratch_bytes<D>(a.use_perm || a.rope);
  static std::atomic<int> occ[2];  // by whether the LDS scratch is allocated
  int per_cu = occ[lds > 0].load(std::memory_order_relaxed);
  CodecArgs b = a;
  unsigned nb = 0;
  if (int e = plan_grid<D>(k, lds, per_cu, b, nb)) return e;
  occ[lds > 0].store(per_cu, std::memory_order_relaxed);
  hipLaunchKernelGGL((encode_kernel<DT, D, BITS, ROT, QUANT, RT, PT, GBT>), dim3(nb), dim3(64 * kWavesPerBlock),
                     lds, s, b);
  return (int)hipGetLastError();
}

template <int ODT, int D, int BITS, int ROT, int QUANT, int PT>
int launch_dec_t(const CodecArgs& a, hipStream_t s) {
  if (a.n_items == 0) return 0;
  const void* k = reinterpret_cast<const void*>(&decode_kernel<ODT, D, BITS, ROT, QUANT, PT>);
  const size_t lds = scratch_bytes<D>(a.use_perm);
  static std::atomic<int> occ[2];  // by whether the LDS scratch is allocated
  int per_cu = occ[lds > 0].load(std::memory_order_relaxed);
  CodecArgs b = a;
  unsigned nb = 0;
  if (int e = plan_grid<D>(k, lds, per_cu, b, nb)) return e;
  occ[lds > 0].store(per_cu, std::memory_order_relaxed);
  hipLaunchKernelGGL((decode_kernel<ODT, D, BITS, ROT, QUANT, PT>), dim3(nb), dim3(64 * kWavesPerBlock),
                     lds, s, b);
  return (int)hipGetLastError();
}

// FWHT + min-max, the hot configurations: RoPE, permutation and group size fixed at
// compile time.
template <int DT, int D, int BITS, int RT, int PT>
int pick_group(const CodecArgs& a, hipStream_t s) {
  switch (a.group_log2) {
    case 5: return launch_enc_t<DT, D, BITS, ROT_FWHT, Q_MINMAX, RT, PT, 5>(a, s);
    case 6: return launch_enc_t<DT, D, BITS, ROT_FWHT, Q_MINMAX, RT, PT, 6>(a, s);
    case 7: return launch_enc_t<DT, D, BITS, ROT_FWHT, Q_MINMAX, RT, PT, 7>(a, s);
    default:
      if constexpr (D == 256) return launch_enc_t<DT, D, BITS, ROT_FWHT, Q_MINMAX, RT, PT, 8>(a, s);
      return (int)hipErrorInvalidValue;
  }
}

template <bool ENC, int DT, int D, int BITS, int ROT, int QUANT>
int pick_feat(const CodecArgs& a, hipStream_t s) {
  if constexpr (ENC) {
    if constexpr (ROT == ROT_FWHT && QUANT == Q_MINMAX) {
      if (a.rope) return a.use_perm ? pick_group<DT, D, BITS, 1, 1>(a, s) : pick_group<DT, D, BITS, 1, 0>(a, s);
      return a.use_perm ? pick_group<DT, D, BITS, 0, 1>(a, s) : pick_group<DT, D, BITS, 0, 0>(a, s);
    } else if constexpr (ROT == ROT_FWHT) {
      if (a.rope)
        return a.use_perm ? launch_enc_t<DT, D, BITS, ROT, QUANT, 1, 1, -1>(a, s)
                          : launch_enc_t<DT, D, BITS, ROT, QUANT, 1, 0, -1>(a, s);
      return a.use_perm ? launch_enc_t<DT, D, BITS, ROT, QUANT, 0, 1, -1>(a, s)
                        : launch_enc_t<DT, D, BITS, ROT, QUANT, 0, 0, -1>(a, s);
    } else {
      return launch_enc_t<DT, D, BITS, ROT, QUANT, -1, -1, -1>(a, s);
    }
  } else {
    if constexpr (ROT == ROT_FWHT) {
      return a.use_perm ? launch_dec_t<DT, D, BITS, ROT, QUANT, 1>(a, s)
                        : launch_dec_t<DT, D, BITS, ROT, QUANT, 0>(a, s);
    } else {
      return launch_dec_t<DT, D, BITS, ROT, QUANT, -1>(a, s);
    }
  }
}

template <bool ENC, int DT, int D, int BITS, int ROT>
int pick_quant(int quant, const CodecArgs& a, hipStream_t s) {
  if (quant == Q_MINMAX) return pick_feat<ENC, DT, D, BITS, ROT, Q_MINMAX>(a, s);
  return pick_feat<ENC, DT, D, BITS, ROT, Q_LLOYD>(a, s);
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

}  // namespace

// One translation unit per (direction, dtype, head_dim) when KVQ_UNIT is 0..11, so
// the kernel instances build in parallel; without KVQ_UNIT every launcher is
// defined here.
#ifndef KVQ_UNIT
#define KVQ_UNIT -1
#endif

#define KVQ_DEFINE_LAUNCH(NAME, UNIT, ENC, DT, D)                                              \
  int NAME(int bits, int rot, int quant, const CodecArgs& a, void* stream) {                   \
    return pick_bits<ENC, DT, D>(bits, rot, quant, a, reinterpret_cast<hipStream_t>(stream));  \
  }

#if KVQ_UNIT == 0 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_encode_f16_d128, 0, true, DT_F16, 128)
const char* device_error_string(int err) { return hipGetErrorString((hipError_t)err); }
#endif
#if KVQ_UNIT == 1 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_encode_f16_d256, 1, true, DT_F16, 256)
#endif
#if KVQ_UNIT == 2 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_encode_bf16_d128, 2, true, DT_BF16, 128)
#endif
#if KVQ_UNIT == 3 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_encode_bf16_d256, 3, true, DT_BF16, 256)
#endif
#if KVQ_UNIT == 4 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_encode_f32_d128, 4, true, DT_F32, 128)
#endif
#if KVQ_UNIT == 5 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_encode_f32_d256, 5, true, DT_F32, 256)
#endif
#if KVQ_UNIT == 6 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_decode_f16_d128, 6, false, DT_F16, 128)
#endif
#if KVQ_UNIT == 7 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_decode_f16_d256, 7, false, DT_F16, 256)
#endif
#if KVQ_UNIT == 8 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_decode_bf16_d128, 8, false, DT_BF16, 128)
#endif
#if KVQ_UNIT == 9 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_decode_bf16_d256, 9, false, DT_BF16, 256)
#endif
#if KVQ_UNIT == 10 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_decode_f32_d128, 10, false, DT_F32, 128)
#endif
#if KVQ_UNIT == 11 || KVQ_UNIT == -1
KVQ_DEFINE_LAUNCH(launch_decode_f32_d256, 11, false, DT_F32, 256)
#endif

}  // namespace kvq
