// HIP kernels of the rotation + low-bit KV-cache codec, written for gfx950 (CDNA4).
//
// Lane layout.  A sub-wavefront of LV = D/32 lanes owns one token-head vector (LV = 4
// at d = 128, 8 at d = 256), so a wave64 holds VPW = 64/LV vectors.  Lane l of a
// vector holds the 32 consecutive channels 32l .. 32l + 31 in slots 0..31.  A lane's
// packed codes are then one contiguous run of 4*bits bytes, so code planes move with a
// single 8/12/16-byte access per lane and the wave covers whole records.
//
// Work.  An item is a tile of VPW consecutive (token, head) columns of one row; a task
// is one tile over a few consecutive rows, and the grid has one wave per task (the
// dispatcher keeps the SIMDs full to the end).  A wave keeps the same columns -- and the
// same RoPE table -- over its rows, with the next item's loads in flight while it
// computes the current one.  Global memory is accessed through buffer descriptors sized
// to what an item may touch, so lanes past the end of a tensor need no branches.
//
// Walsh-Hadamard.  The channel index splits into 5 in-lane bits (slots) and 2 or 3
// lane bits.  In-lane butterflies are plain VALU adds; lane-bit butterflies are a
// v_fmac with a DPP quad_perm operand (lane xor 1, xor 2) or a ds_swizzle partner
// (xor 4): own + m * partner with m = +-1 per lane.  With m = -1 on the lane whose bit
// is set, lane l ends up holding (-1)^popcount(l) times the true coefficient; that sign
// is folded into the quantization scale.  With m = +1 there and inputs pre-multiplied
// by (-1)^popcount(l), the lanes hold the true coefficients (used by the decoder).
//
// LDS holds parameters (RoPE frequencies, SO(4) matrices) and per-wave staging: the
// cos/sin table of the tokens of the wave's current tile, the channel permutation (a
// gather or scatter of 32 values per lane through one row per vector), and the
// decoder's output, which is written per lane and read back so that every global store
// of the wave covers 1 KiB of contiguous output.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "kvq_internal.h"

namespace kvq {
namespace {

enum { DT_F16 = 0, DT_BF16 = 1, DT_F32 = 2 };
enum { ROT_NONE = 0, ROT_FWHT = 1, ROT_SO4 = 2, ROT_DENSE = 3, ROT_ROTOR = 4 };
enum { Q_MINMAX = 0, Q_LLOYD = 1 };

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x3_t __attribute__((ext_vector_type(3)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

template <int D>
struct Geo {
  static constexpr int LV = D / 32;             // lanes per vector
  static constexpr int LVB = (LV == 4) ? 2 : 3;  // log2(LV)
  static constexpr int VPW = 64 / LV;            // vectors per wave
};

// Per-wave LDS staging: one row per vector of the wave.  A row holds the vector as
// floats (D * 4 bytes) plus 16 bytes of padding, which staggers the rows across banks.
template <int D>
constexpr int row_bytes() {
  return D * 4 + 16;
}
template <int D>
constexpr int stage_wave_bytes() {
  return Geo<D>::VPW * row_bytes<D>();
}
// Decoder staging rows hold a vector in the output type (D * bytes + 16 of padding).
template <int D, int ODT>
constexpr int dec_row_bytes() {
  return D * (ODT == DT_F32 ? 4 : 2) + 16;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_f32*)p;
}
__device__ __forceinline__ float lds_ld(uint32_t addr) { return *(const lds_f32*)(uintptr_t)addr; }
__device__ __forceinline__ void lds_st(uint32_t addr, float v) { *(lds_f32*)(uintptr_t)addr = v; }
__device__ __forceinline__ void lds_st16(uint32_t addr, uint16_t v) {
  *(__attribute__((address_space(3))) uint16_t*)(uintptr_t)addr = v;
}
__device__ __forceinline__ u32x4_t lds_ld4(uint32_t addr) { return *(const lds_u32x4*)(uintptr_t)addr; }
__device__ __forceinline__ void lds_st4(uint32_t addr, u32x4_t v) { *(lds_u32x4*)(uintptr_t)addr = v; }

// Raw buffer accesses: a wave-uniform descriptor (base address and size in bytes, in
// SGPRs) plus a per-lane byte offset.  A lane whose access starts at or beyond the size
// reads zeros and its store is dropped.  Sizing each descriptor to the part of the tensor
// an item may touch makes lanes past the end of a tensor (and the prefetch after a wave's
// last item, with size 0) harmless without any branch or per-lane select, so the hot
// loops stay straight-line and the next item's loads stay in flight while the current
// item is computed.  The sizes are whole vectors (or a whole row of the input, whose
// strides are multiples of 16 bytes), so each lane's access lies wholly inside or wholly
// outside its descriptor.
typedef __amdgpu_buffer_rsrc_t buf_t;
constexpr int kBufWord3 = 0x00020000;  // descriptor word 3 for untyped access on gfx9
constexpr int kNT = 2;                 // cache-policy bit: non-temporal (streamed data:
                                       // code records and decoded output, measured 3 %
                                       // faster over a round trip; the encoder's input
                                       // loads stay temporal, see load_row)
constexpr int kSC1 = 16;               // cache-policy bit: system scope (sc1); with kNT on
                                       // the decoders' output stores, measured 2 % faster
__device__ __forceinline__ buf_t make_buf(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kBufWord3);
}
// The same for the planes and output of one item (at most 16 KiB, so no clamp).
__device__ __forceinline__ buf_t make_buf_item(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}

// Orders this wave's LDS accesses before and after the call (LDS ops of one wave are
// executed in order; this keeps the compiler from moving them across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// cross-lane primitives
// ---------------------------------------------------------------------------
#define KVQ_QP1 " quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
#define KVQ_QP2 " quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"

// v <- partner(v) * m + v for 8 values, partner = lane xor 1.  The leading s_nop gives
// the 2 wait states a DPP read needs after a VALU write of its operand, since the compiler
// does not look inside the asm (no VALU instruction in these kernels writes EXEC, which
// would need 5).
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
// Sums over 8 and 16 lanes that finish what add_x1 and add_x2 began: the value is then equal
// within each quad, so the partner across the half-row mirror (lane 7 - i of 8) or the row
// mirror (15 - i of 16) holds what lane i ^ 4 or i ^ 8 holds, and every lane gets the same
// sum in the same order as an xor butterfly.  DPP, without the LDS round trip of ds_swizzle.
__device__ __forceinline__ float add_half_mirror(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float add_row_mirror(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
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

// Bitwise OR over the LV lanes of a vector (every lane gets the result).
template <int LV>
__device__ __forceinline__ uint32_t vec_or(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // lane xor 1
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // lane xor 2
  if constexpr (LV == 8) v |= (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F);
  return v;
}

__device__ __forceinline__ float lane_sign(int l) {
  return (__builtin_popcount(l) & 1) ? -1.0f : 1.0f;
}

// ---------------------------------------------------------------------------
// Walsh-Hadamard, unnormalised, on the 32 slots of a lane (from slot bit FIRST on)
// plus the lane bits, with per-lane multipliers m1, m2, m4 for the lane stages.
// ---------------------------------------------------------------------------
template <int LV, int FIRST = 0>
__device__ __forceinline__ void fwht_lane(float* v, float m1, float m2, float m4) {
#pragma unroll
  for (int hb = 1 << FIRST; hb < 32; hb <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i & hb) continue;
      const float a = v[i], b = v[i + hb];
      v[i] = a + b;
      v[i + hb] = a - b;
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) fmac_x1(v + 8 * k, m1);
#pragma unroll
  for (int k = 0; k < 4; ++k) fmac_x2(v + 8 * k, m2);
  if constexpr (LV == 8) {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(swz_x4(v[i]), m4, v[i]);
  }
}

// ---------------------------------------------------------------------------
// dtype conversions
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) { return f16_bits(a) | (f16_bits(b) << 16); }
__device__ __forceinline__ float f16_value(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// fp16 with directed rounding, from the conversion that rounds toward zero: for x < 0 an
// inexact result moves one step away from zero (down), for x >= 0 it is already rounded
// down.  x must not be -0 (the callers add +0 first).
__device__ __forceinline__ uint32_t f16_round_down(float x) {
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x, 0.0f));  // high half 0
  const float back = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  return h + ((back != x && x < 0.0f) ? 1u : 0u);
}
// The same rounded up, for x >= 0 (a scale): an inexact result moves one step up.
__device__ __forceinline__ uint32_t f16_round_up_nonneg(float x) {
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x, 0.0f));
  const float back = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  return h + (back != x ? 1u : 0u);
}

// One lane's 32 channels of one vector as stored: 4 x 16 bytes for 16-bit types,
// 8 x 16 bytes for float.
template <int DT>
struct RawRow {
  static constexpr int NW = (DT == DT_F32) ? 8 : 4;
  u32x4_t w[NW];
};

// Plain (temporal) loads: the four 16-byte loads of a lane hit the same cache lines as
// its neighbours' (each wave instruction covers a 16-byte slice of every 64-byte lane
// run), and with non-temporal hints the lines were fetched from HBM more than once.
template <int DT>
__device__ __forceinline__ void load_row(RawRow<DT>& raw, const char* p) {
#pragma unroll
  for (int k = 0; k < RawRow<DT>::NW; ++k) raw.w[k] = reinterpret_cast<const u32x4_t*>(p)[k];
}
template <int DT>
__device__ __forceinline__ void load_row(RawRow<DT>& raw, buf_t b, uint32_t off) {
#pragma unroll
  for (int k = 0; k < RawRow<DT>::NW; ++k) raw.w[k] = __builtin_amdgcn_raw_buffer_load_b128(b, off + 16u * k, 0, 0);
}

template <int DT>
__device__ __forceinline__ void widen_row(const RawRow<DT>& raw, float* v) {
#pragma unroll
  for (int k = 0; k < RawRow<DT>::NW; ++k) {
    const uint32_t ws[4] = {raw.w[k].x, raw.w[k].y, raw.w[k].z, raw.w[k].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == DT_F32) {
        v[4 * k + i] = __uint_as_float(ws[i]);
      } else if constexpr (DT == DT_BF16) {
        v[8 * k + 2 * i] = __uint_as_float(ws[i] << 16);
        v[8 * k + 2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
      } else {
        v[8 * k + 2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws[i] & 0xffffu));
        v[8 * k + 2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws[i] >> 16));
      }
    }
  }
}

// Slots 8c .. 8c + 7 of a raw row, widened.
template <int DT>
__device__ __forceinline__ void widen_chunk(const RawRow<DT>& raw, int c, float* t) {
  if constexpr (DT == DT_F32) {
    const u32x4_t a = raw.w[2 * c], b = raw.w[2 * c + 1];
    t[0] = __uint_as_float(a.x); t[1] = __uint_as_float(a.y); t[2] = __uint_as_float(a.z); t[3] = __uint_as_float(a.w);
    t[4] = __uint_as_float(b.x); t[5] = __uint_as_float(b.y); t[6] = __uint_as_float(b.z); t[7] = __uint_as_float(b.w);
  } else {
    const uint32_t ws[4] = {raw.w[c].x, raw.w[c].y, raw.w[c].z, raw.w[c].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == DT_BF16) {
        t[2 * i] = __uint_as_float(ws[i] << 16);
        t[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
      } else {
        t[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws[i] & 0xffffu));
        t[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws[i] >> 16));
      }
    }
  }
}

// Widen a 16-bit row and apply the first two Walsh-Hadamard stages (slot bits 0 and 1)
// at once: each group of 4 channels (two dwords p, r) gives
//   x0+x1+x2+x3, x0-x1+x2-x3, x0+x1-x2-x3, x0-x1-x2+x3
// from two v_dot2 of p (x0+x1, x0-x1) and four v_dot2 of r with those as addends.
// Eight outputs (two groups of 4 channels, dwords X Y and Z W) with the three-address
// dot instruction OP: the builtins select the accumulating two-address form, which costs
// a copy of every partial sum used twice and a zeroed register for every zero addend.
// The 4 zero-addend dots go first, so every dependent dot reads a result at least 3
// instructions old; the closing s_nop 2 gives the 3 wait states a dot result needs
// before other VALU instructions read it.
#define KVQ_H4_BLOCK(OP, o, X, Y, Z, W)                                                           \
  {                                                                                               \
    float s0, d0, s1, d1;                                                                         \
    asm volatile(OP " %8, %12, %16, 0\n\t" OP " %9, %12, %17, 0\n\t" OP " %10, %14, %16, 0\n\t"  \
                 OP " %11, %14, %17, 0\n\t" OP " %0, %13, %16, %8\n\t" OP " %1, %13, %17, %9\n\t" \
                 OP " %2, %13, %18, %8\n\t" OP " %3, %13, %19, %9\n\t" OP " %4, %15, %16, %10\n\t"\
                 OP " %5, %15, %17, %11\n\t" OP " %6, %15, %18, %10\n\t" OP " %7, %15, %19, %11\n\t" \
                 "s_nop 2"                                                                        \
                 : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),  \
                   "=&v"(o[6]), "=&v"(o[7]), "=&v"(s0), "=&v"(d0), "=&v"(s1), "=&v"(d1)           \
                 : "v"(X), "v"(Y), "v"(Z), "v"(W), "s"(c11), "s"(c1m), "s"(cmm), "s"(cm1));      \
  }
template <int DT>
__device__ __forceinline__ void widen_row_h4(const RawRow<DT>& raw, float* v) {
  static_assert(DT != DT_F32, "16-bit inputs only");
  // packed (+-1, +-1) pairs: low half multiplies the even channel
  constexpr uint32_t P1 = (DT == DT_BF16) ? 0x3F80u : 0x3C00u, M1 = P1 | 0x8000u;
  const uint32_t c11 = P1 | P1 << 16, c1m = P1 | M1 << 16, cmm = M1 | M1 << 16, cm1 = M1 | P1 << 16;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float* o = v + 8 * k;
    if constexpr (DT == DT_BF16) {
      KVQ_H4_BLOCK("v_dot2_f32_bf16", o, raw.w[k].x, raw.w[k].y, raw.w[k].z, raw.w[k].w)
    } else {
      KVQ_H4_BLOCK("v_dot2_f32_f16", o, raw.w[k].x, raw.w[k].y, raw.w[k].z, raw.w[k].w)
    }
  }
}

// ---------------------------------------------------------------------------
// parameter staging
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

// cos and sin of phi = pos * theta.  The angle (up to ~1e5 rad) and its quadrant
// reduction phi = k*pi/2 + r, |r| <= pi/4, are evaluated in float64 (two-term Cody-Waite
// split of pi/2, exact products for k < 2^31); sin r and cos r then come from their
// Taylor polynomials in float32 (terms up to r^9 / r^10; truncation below 2e-9 for
// |r| <= pi/4), within about 2 ulp of the correctly rounded float.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, double theta, float* c, float* s) {
  constexpr double kTwoOverPi = 0.63661977236758138;
  constexpr double kPio2Hi = 1.570796012878418;       // pi/2 truncated to 22 bits
  constexpr double kPio2Lo = 3.139164786504813e-07;   // pi/2 - kPio2Hi (rounded)
  const double phi = (double)pos * theta;
  const double k = rint(phi * kTwoOverPi);
  double rd = fma(-k, kPio2Hi, phi);
  rd = fma(-k, kPio2Lo, rd);
  const float r = (float)rd, r2 = r * r;
  // sin r = r (1 - r2/3! + r2^2/5! - ...), cos r = 1 - r2/2! + r2^2/4! - ...
  float sn = 1.0f / 362880.0f;                     // 1/9!
  sn = __builtin_fmaf(sn, -r2, 1.0f / 5040.0f);
  sn = __builtin_fmaf(sn, -r2, 1.0f / 120.0f);
  sn = __builtin_fmaf(sn, -r2, 1.0f / 6.0f);
  sn = __builtin_fmaf(sn, -r2, 1.0f);
  sn *= r;
  float cs = 1.0f / 3628800.0f;                    // 1/10!
  cs = __builtin_fmaf(cs, -r2, 1.0f / 40320.0f);
  cs = __builtin_fmaf(cs, -r2, 1.0f / 720.0f);
  cs = __builtin_fmaf(cs, -r2, 1.0f / 24.0f);
  cs = __builtin_fmaf(cs, -r2, 0.5f);
  cs = __builtin_fmaf(cs, -r2, 1.0f);
  const int quad = (int)((int64_t)k & 3);
  const float oc = (quad & 1) ? sn : cs, os = (quad & 1) ? cs : sn;
  *c = (quad == 1 || quad == 2) ? -oc : oc;
  *s = (quad >= 2) ? -os : os;
}

// ---------------------------------------------------------------------------
// work walk shared by both kernels
// ---------------------------------------------------------------------------
// The lane's vector in a tile: column col = tile*VPW + q = (t0 + dtok) * heads + h.
// The encoder's input address is a wave-uniform base (row, t0) plus a 32-bit lane
// offset; the host bounds 16 token strides plus a head span below 2^31 bytes.
struct LaneTile {
  int64_t tile, t0;
  int64_t pos;     // pos_offset + token of the lane's vector
  int32_t h;       // head of the lane's vector
  int32_t dtok;    // token - t0
  int32_t valid;   // col < tokens * heads (0 / 1; a full word keeps the struct in registers)
  int32_t pad;
};

// n / d for 0 <= n < 2^31 with the host's constants for d
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  return (uint32_t)(((uint64_t)n * f.mul) >> f.shift);
}

// (columns stay below 2^31: tokens * heads is checked on the host)
template <int VPW>
__device__ __forceinline__ LaneTile lane_tile(const CodecArgs& a, int64_t tile, int q) {
  LaneTile lt;
  lt.tile = tile;
  const uint32_t heads = (uint32_t)a.heads;
  const uint32_t col0 = (uint32_t)tile * VPW;
  const uint32_t t0 = fdiv(col0, a.div_heads);
  const uint32_t hq = col0 - t0 * heads + (uint32_t)q;  // < heads + 64
  const uint32_t dt = fdiv(hq, a.div_heads);
  lt.t0 = t0;
  lt.dtok = (int32_t)dt;
  lt.h = (int32_t)(hq - dt * heads);
  lt.pos = a.pos_offset + (int64_t)(t0 + dt);
  lt.valid = ((int64_t)col0 + q < a.tokens * a.heads) ? 1 : 0;
  lt.pad = 0;
  return lt;
}

// A wave's walk over its task.  Encoder: tile wid % n_tiles over the rows
// [k * (wid / n_tiles), min(k * (wid / n_tiles + 1), rows)), so a wave keeps its tile (and
// RoPE table) down its rows.  Decoder: tiles [k * (wid % n_tblk), ...) of row
// wid / n_tblk, so a wave's output is one contiguous run.  k = task_len.  The grid holds
// every task, so the hardware dispatcher keeps the SIMDs full until the end.
struct Walk {
  int64_t tile, r;  // current item
  int64_t end;      // one past the task's last row (encoder) or tile (decoder)
};

// (wave ids stay below 2^31: the launcher checks the number of tasks)
__device__ __forceinline__ bool walk_first_rows(const CodecArgs& a, uint32_t wid, Walk& w) {
  const uint32_t run = fdiv(wid, a.div_task);
  w.tile = wid - run * (uint32_t)a.n_tiles;
  w.r = (int64_t)run * a.task_len;
  w.end = min(w.r + a.task_len, a.rows);
  return w.r < a.rows;
}
__device__ __forceinline__ bool walk_next_rows(Walk& w) { return ++w.r < w.end; }

__device__ __forceinline__ bool walk_first_tiles(const CodecArgs& a, uint32_t wid, Walk& w) {
  const uint32_t row = fdiv(wid, a.div_task);
  w.r = row;
  w.tile = (int64_t)(wid - row * (uint32_t)a.n_tblk) * a.task_len;
  w.end = min(w.tile + a.task_len, a.n_tiles);
  return w.r < a.rows;
}
__device__ __forceinline__ bool walk_next_tiles(Walk& w) { return ++w.tile < w.end; }

// ---------------------------------------------------------------------------
// bit-packing of a lane's 32 codes (4*BITS bytes, code i at bits BITS*i)
// ---------------------------------------------------------------------------
template <int BITS>
struct LaneCodes {
  static constexpr int NW = BITS;  // 32-bit words: 32 codes * BITS bits / 32
  uint32_t w[NW];
};

template <int BITS>
__device__ __forceinline__ void store_lane_codes(buf_t b, uint32_t off, const LaneCodes<BITS>& c) {
  if constexpr (BITS == 2) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{c.w[0], c.w[1]}, b, off, 0, kNT);
  } else if constexpr (BITS == 4) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{c.w[0], c.w[1], c.w[2], c.w[3]}, b, off, 0, kNT);
  } else {
    __builtin_amdgcn_raw_buffer_store_b96(u32x3_t{c.w[0], c.w[1], c.w[2]}, b, off, 0, kNT);
  }
}
template <int BITS>
__device__ __forceinline__ void store_lane_codes(uint8_t* p, const LaneCodes<BITS>& c) {
  if constexpr (BITS == 2) {
    u32x2_t v = {c.w[0], c.w[1]};
    *reinterpret_cast<u32x2_t*>(p) = v;
  } else if constexpr (BITS == 4) {
    u32x4_t v = {c.w[0], c.w[1], c.w[2], c.w[3]};
    *reinterpret_cast<u32x4_t*>(p) = v;
  } else {
    uint32_t* d = reinterpret_cast<uint32_t*>(p);
    d[0] = c.w[0];
    d[1] = c.w[1];
    d[2] = c.w[2];
  }
}

template <int BITS>
__device__ __forceinline__ void load_lane_codes(buf_t b, uint32_t off, LaneCodes<BITS>& c) {
  if constexpr (BITS == 2) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(b, off, 0, kNT);
    c.w[0] = v.x;
    c.w[1] = v.y;
  } else if constexpr (BITS == 4) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(b, off, 0, kNT);
    c.w[0] = v.x;
    c.w[1] = v.y;
    c.w[2] = v.z;
    c.w[3] = v.w;
  } else {
    const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(b, off, 0, kNT);
    c.w[0] = v.x;
    c.w[1] = v.y;
    c.w[2] = v.z;
  }
}

// Code i of a lane (0 <= i < 32).
template <int BITS>
__device__ __forceinline__ uint32_t code_at(const LaneCodes<BITS>& c, int i) {
  if constexpr (BITS == 3) {
    const int bit = 3 * i, w = bit >> 5, sh = bit & 31;
    if (sh <= 29) return (c.w[w] >> sh) & 7u;
    return ((c.w[w] >> sh) | (c.w[w + 1] << (32 - sh))) & 7u;
  } else {
    const int bit = BITS * i;
    return (c.w[bit >> 5] >> (bit & 31)) & ((1u << BITS) - 1u);
  }
}

// Per-wave encoder staging: permutation rows (when a permutation is used), then the
// RoPE table of the wave's tile: trig_rows rows of D/2 (cos, sin) float pairs.
// Encoder permutation rows: lane l's 32 floats at byte 128 l of a row of D * 4 + 16 bytes,
// its 16-byte piece k at 16 ((k + l) mod 8): the rotation puts the lanes of a vector on
// different banks, so the rows need no padding between lanes.  With it a block's staging is
// 40 KB at d = 128, 4 blocks per CU: 2 % faster for the RoPE + permutation encoder than 3
// blocks of 160-byte lane pitches (unrotated 128-byte pitches: 7 % slower).
template <int D>
constexpr int enc_pitch() {
  return 128;
}
template <int D>
constexpr int enc_row() {
  return D * 4 + 16;
}
template <int D>
__device__ __forceinline__ uint32_t enc_perm_bytes(bool perm) {
  return perm ? (uint32_t)(Geo<D>::VPW * enc_row<D>()) : 0u;
}
// RoPE table: a token's D/2 (cos, sin) pairs, the 16 pairs lane l reads at byte l * kTrigLane,
// its 16-byte piece k (pairs 2k, 2k + 1) at 16 ((k + l) mod 8), the same rotation as the rows
// (16-byte LDS reads are served 16 lanes at a time on 64 banks of 4 bytes).
constexpr int kTrigLane = 128;
template <int D>
constexpr int trig_row() {
  return Geo<D>::LV * kTrigLane;
}
template <int D>
__device__ __host__ inline size_t enc_wave_bytes(bool perm, bool rope, int trig_rows) {
  return (perm ? (size_t)(Geo<D>::VPW * enc_row<D>()) : 0) + (rope ? (size_t)trig_rows * trig_row<D>() : 0);
}

// ---------------------------------------------------------------------------
// quantization of a lane's 32 values (shared by the encoders)
// ---------------------------------------------------------------------------
// Norm separation of the Lloyd-Max path (IsoQuant page, section 3.1): rho = |v| over the
// vector's LV lanes, with an exact power-of-two pre-scale by the largest |v_i| so that the sum
// of squares neither underflows nor overflows; v becomes v / (rho + 1e-6).  Returns rho.
template <int LV>
__device__ __forceinline__ float norm_separate(float* v) {
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
  return rho;
}

// Min-max quantization of a lane's 32 values whose true coefficients are A * v (for A < 0 min
// and max swap).  A group covers 2^LB whole lanes (LB = log2 G - 5).  Returns the group's zero
// (rounded down) and scale = (max - zero) / (2^b - 1) (rounded up) as fp16 bits, the same in
// every lane of the group, and the codes q = rint((A v - zero) / scale), nearest-even.  RESID:
// one residual step first makes the quotient correctly rounded (unrotated 16-bit data sit on
// the zero/scale grid, so exact half-way quotients are common).
template <int BITS, bool RESID>
__device__ __forceinline__ void minmax_codes_lane(const float* v, float A, int LB, uint32_t& zb_out, uint32_t& sb_out,
                                                  LaneCodes<BITS>& cw) {
  float lo = fminf(fminf(v[0], v[1]), v[2]), hi = fmaxf(fmaxf(v[0], v[1]), v[2]);
#pragma unroll
  for (int i = 3; i < 31; i += 2) {
    lo = fminf(fminf(lo, v[i]), v[i + 1]);
    hi = fmaxf(fmaxf(hi, v[i]), v[i + 1]);
  }
  lo = fminf(lo, v[31]);
  hi = fmaxf(hi, v[31]);
  float mn = (A > 0.0f) ? lo * A : hi * A;
  float mx = (A > 0.0f) ? hi * A : lo * A;
  if (LB >= 1) { mn = min_x1(mn); mx = max_x1(mx); }
  if (LB >= 2) { mn = min_x2(mn); mx = max_x2(mx); }
  if (LB >= 3) { mn = fminf(mn, swz_x4(mn)); mx = fmaxf(mx, swz_x4(mx)); }
  // "+ 0.0f" turns a -0 (all-zero group, negated lanes) into +0
  const uint32_t zb = f16_round_down(mn + 0.0f);
  const float z = f16_value(zb);
  constexpr float kInvLevels = 1.0f / (float)((1 << BITS) - 1);
  const uint32_t sb = f16_round_up_nonneg((mx - z) * kInvLevels + 0.0f);
  const float sc = f16_value(sb);
  zb_out = zb;
  sb_out = sb;
  const float iv = (sc > 0.0f) ? __builtin_amdgcn_rcpf(sc) : 0.0f;
  float tv[32];
  if constexpr (RESID) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float d = __builtin_fmaf(v[i], A, -z);
      const float t0 = d * iv;
      tv[i] = (sc > 0.0f) ? __builtin_fmaf(__builtin_fmaf(-t0, sc, d), iv, t0) : 0.0f;
    }
  } else {
    const float Ai = A * iv, c0 = -z * iv;
#pragma unroll
    for (int i = 0; i < 32; ++i) tv[i] = __builtin_fmaf(v[i], Ai, c0);
  }
  if constexpr (BITS == 3) {
    // q = rint(t) via 1.5 * 2^23: the sum rounds t to an integer in the low mantissa bits
    // (bit pattern 0x4B400000 + q, since -eps <= t <= 2^b - 1 + eps)
    constexpr float kMagic = 12582912.0f;
#pragma unroll
    for (int w = 0; w < 3; ++w) cw.w[w] = 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t cq = __float_as_uint(tv[i] + kMagic) - 0x4B400000u;
      const int bit = 3 * i, w = bit >> 5, sh = bit & 31;
      cw.w[w] |= cq << sh;
      if (sh > 29) cw.w[w + 1] |= cq >> (32 - sh);
    }
  } else {
    // v_cvt_pk_u8_f32 (round to nearest even, clamped at 0) writes code k + ND j into byte j of
    // dword D_k; the word is D_0 + D_1 << BITS + ... (each byte's code lands on its own field)
    constexpr int PER = 32 / BITS;  // codes per word
    constexpr int ND = PER / 4;     // dwords D_k per word
#pragma unroll
    for (int w = 0; w < BITS; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int k = ND - 1; k >= 0; --k) {
        uint32_t d = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) d = __builtin_amdgcn_cvt_pk_u8_f32(tv[PER * w + k + ND * j], j, d);
        word = (word << BITS) + d;
      }
      cw.w[w] = word;
    }
  }
}

// Lloyd-Max codes of a lane's 32 values (true coefficients A * v): q = #{k : z > tau_k} against
// the 2^b - 1 midpoints tau.
template <int BITS>
__device__ __forceinline__ void lloyd_codes_lane(const float* v, float A, const float* tau, LaneCodes<BITS>& cw) {
  constexpr int NT = (1 << BITS) - 1;
#pragma unroll
  for (int w = 0; w < BITS; ++w) cw.w[w] = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float z = v[i] * A;
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < NT; ++k) c += (z > tau[k]) ? 1u : 0u;
    const int bit = BITS * i, w = bit >> 5, sh = bit & 31;
    cw.w[w] |= c << sh;
    if (BITS == 3 && sh > 29) cw.w[w + 1] |= c >> (32 - sh);
  }
}

// ---------------------------------------------------------------------------
// RotorQuant's 3-D rotors (the baseline of the IsoQuant page, section 1)
// ---------------------------------------------------------------------------
// Block b (channels 3b .. 3b + 2, b < D / 3) turns by the rotor of unit quaternion r_b, the
// sandwich product r (0, v) r*, as its 3x3 matrix; a 2-channel tail turns by (cos t, sin t); a
// 1-channel tail stays.  Table in LDS: 12 floats per block (rows of 3, each padded to 4), then
// the tail's (cos t, sin t).  Built from CodecArgs.quat: r_b at quat[4 b], then (cos t, sin t).
template <int D>
__device__ void build_rotor_table(const float* rq, float* tab) {
  constexpr int NB = D / 3;
  for (int b = threadIdx.x; b <= NB; b += blockDim.x) {
    float* m = tab + 12 * b;
    if (b == NB) {
      m[0] = rq[4 * NB];
      m[1] = rq[4 * NB + 1];
      continue;
    }
    const float w = rq[4 * b], x = rq[4 * b + 1], y = rq[4 * b + 2], z = rq[4 * b + 3];
    // homogeneous form: equals r (0, v) r* for any r (|r|^2 times the rotation)
    m[0] = w * w + x * x - y * y - z * z; m[1] = 2.0f * (x * y - w * z); m[2] = 2.0f * (x * z + w * y); m[3] = 0.0f;
    m[4] = 2.0f * (x * y + w * z); m[5] = w * w - x * x + y * y - z * z; m[6] = 2.0f * (y * z - w * x); m[7] = 0.0f;
    m[8] = 2.0f * (x * z - w * y); m[9] = 2.0f * (y * z + w * x); m[10] = w * w - x * x - y * y + z * z; m[11] = 0.0f;
  }
}

// The rotation (INV: its inverse, the transposed blocks and the tail turned back) of a vector
// held as 32 values per lane (lane l: channels 32 l ..), through the vector's LDS row of
// contiguous floats: lane l turns blocks 11 l .. 11 l + 10 (channels 33 l ..) in place, one
// block at a time (each lane reads and writes only its own channels there), the last lane also
// the tail; then every lane reads its 32 channels back.  3-D blocks do not align with the
// lanes' 32 channels, hence the row.
template <int D, bool INV>
__device__ __forceinline__ void rotor_lane(float* v, uint32_t row, int l, uint32_t tab) {
  constexpr int LV = D / 32, NB = D / 3, TAIL = D % 3;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    lds_st4(row + 128u * l + 16u * k, u32x4_t{__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]),
                                             __float_as_uint(v[4 * k + 2]), __float_as_uint(v[4 * k + 3])});
  wave_lds_sync();
  const int nblk = min(11, NB - 11 * l);  // the lane's whole blocks
  const uint32_t span = row + 132u * (uint32_t)l;
  const uint32_t mtab = tab + 528u * (uint32_t)l;  // block 11 l
#pragma unroll 1
  for (int j = 0; j < nblk; ++j) {
    const uint32_t p = span + 12u * (uint32_t)j, m = mtab + 48u * (uint32_t)j;
    const float a0 = lds_ld(p), a1 = lds_ld(p + 4u), a2 = lds_ld(p + 8u);
    const u32x4_t r0 = lds_ld4(m), r1 = lds_ld4(m + 16u), r2 = lds_ld4(m + 32u);
    float z0, z1, z2;
    if constexpr (!INV) {
      z0 = __builtin_fmaf(__uint_as_float(r0.x), a0, __builtin_fmaf(__uint_as_float(r0.y), a1, __uint_as_float(r0.z) * a2));
      z1 = __builtin_fmaf(__uint_as_float(r1.x), a0, __builtin_fmaf(__uint_as_float(r1.y), a1, __uint_as_float(r1.z) * a2));
      z2 = __builtin_fmaf(__uint_as_float(r2.x), a0, __builtin_fmaf(__uint_as_float(r2.y), a1, __uint_as_float(r2.z) * a2));
    } else {
      z0 = __builtin_fmaf(__uint_as_float(r0.x), a0, __builtin_fmaf(__uint_as_float(r1.x), a1, __uint_as_float(r2.x) * a2));
      z1 = __builtin_fmaf(__uint_as_float(r0.y), a0, __builtin_fmaf(__uint_as_float(r1.y), a1, __uint_as_float(r2.y) * a2));
      z2 = __builtin_fmaf(__uint_as_float(r0.z), a0, __builtin_fmaf(__uint_as_float(r1.z), a1, __uint_as_float(r2.z) * a2));
    }
    lds_st(p, z0);
    lds_st(p + 4u, z1);
    lds_st(p + 8u, z2);
  }
  if constexpr (TAIL == 2) {
    if (l == LV - 1) {
      const uint32_t p = row + 4u * (3 * NB);
      const float c = lds_ld(tab + 48u * NB), sn = INV ? -lds_ld(tab + 48u * NB + 4u) : lds_ld(tab + 48u * NB + 4u);
      const float a0 = lds_ld(p), a1 = lds_ld(p + 4u);
      lds_st(p, __builtin_fmaf(c, a0, -sn * a1));
      lds_st(p + 4u, __builtin_fmaf(sn, a0, c * a1));
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const u32x4_t w = lds_ld4(row + 128u * l + 16u * k);
    v[4 * k] = __uint_as_float(w.x);
    v[4 * k + 1] = __uint_as_float(w.y);
    v[4 * k + 2] = __uint_as_float(w.z);
    v[4 * k + 3] = __uint_as_float(w.w);
  }
  wave_lds_sync();  // the row is free again
}

// ---------------------------------------------------------------------------
// ENCODE
// ---------------------------------------------------------------------------
// RT / PT: RoPE / permutation off (0), on (1) or read from the arguments (-1).
// GBT: log2 of the min-max group size, or -1 to read it from the arguments.  The hot
// configurations get compile-time values; the rest share run-time variants.
// AP: append mode (one token per row at the row's own position, into a cache of cap
// slots per row); one item per wave, so each wave builds its RoPE table for its row.
template <int DT, int D, int BITS, int ROT, int QUANT, int RT, int PT, int GBT, int AP = 0>
__global__ void __launch_bounds__(64 * kWavesPerBlock) encode_kernel(const CodecArgs a) {
  using G = Geo<D>;
  constexpr int LV = G::LV, VPW = G::VPW;
  constexpr bool ROPE_ANY = RT != 0, PERM_ANY = PT != 0;
  const bool ROPE = (RT < 0) ? (a.rope != 0) : (RT == 1);
  const bool PERM = (PT < 0) ? (a.use_perm != 0) : (PT == 1);
  extern __shared__ float s_stage[];
  __shared__ double s_theta[ROPE_ANY ? D / 2 : 1];
  __shared__ float s_mat[ROT == ROT_SO4 ? (D / 4) * 16 : 1];
  __shared__ __attribute__((aligned(16))) float s_rtab[ROT == ROT_ROTOR ? (D / 3 + 1) * 12 : 4];
  __shared__ __attribute__((aligned(16))) uint16_t s_goff[PERM_ANY ? D : 8];
  // dynamic codebook: 1 / scale and the wide-channel rank of each rotated channel
  __shared__ float s_cinv[QUANT == Q_LLOYD ? D : 1];
  __shared__ uint8_t s_rank[QUANT == Q_LLOYD ? D : 1];

  const int tid = threadIdx.x;
  if constexpr (QUANT == Q_LLOYD) {
    if (a.dyn)
      for (int j = tid; j < D; j += blockDim.x) {
        s_cinv[j] = 1.0f / a.chan_scale[j];
        s_rank[j] = a.wide_rank[j];
      }
  }
  if constexpr (PERM_ANY) {
    // byte offset of channel perm[j] in a staging row, for the gather
    if (PERM)
      for (int j = tid; j < D; j += blockDim.x) {
        const uint32_t p = a.perm[j];
        s_goff[j] = (uint16_t)((p >> 5) * (uint32_t)enc_pitch<D>() + 16u * ((((p & 31u) >> 2) + (p >> 5)) & 7u) + 4u * (p & 3u));
      }
  }
  if constexpr (ROPE_ANY) {
    if (ROPE)
      for (int i = tid; i < D / 2; i += blockDim.x)
        s_theta[i] = exp2(-(2.0 * (double)i / (double)D) * a.rope_log2_base);
  }
  if constexpr (ROT == ROT_SO4) {
    for (int b = tid; b < D / 4; b += blockDim.x) build_so4(&a.quat[8 * b], &s_mat[16 * b]);
  }
  if constexpr (ROT == ROT_ROTOR) build_rotor_table<D>(a.quat, s_rtab);
  // block-shared parameters ready; the barrier also starts the block's four waves (adjacent
  // tiles) together, which measured about 2 % faster even where there are no parameters
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const uint32_t wid = blockIdx.x * kWavesPerBlock + (uint32_t)wave;
  Walk wk;
  if (!walk_first_rows(a, wid, wk)) return;  // wave-uniform; no barrier follows
  // append: the position of the wave's row (its only item)
  const int64_t prow = AP ? a.row_pos[wk.r] : 0;

  const int q = lane / LV, l = lane % LV;
  const int64_t ncols = a.tokens * a.heads;
  constexpr int ES = (DT == DT_F32) ? 4 : 2;
  constexpr int CB = D * BITS / 8;  // code bytes per vector

  // 16-bit input straight into the transform: widen fused with two butterfly stages
  constexpr bool FUSED = (DT != DT_F32) && RT == 0 && PT == 0 && (QUANT == Q_MINMAX) && (ROT == ROT_FWHT);

  // per-wave staging: permutation rows, then the RoPE table
  // (the rotor also stages each vector, in the permutation rows)
  const bool STAGE = PERM || ROT == ROT_ROTOR;
  const uint32_t wave_addr =
      lds_addr(s_stage) + (uint32_t)(wave * enc_wave_bytes<D>(STAGE, ROPE, a.trig_rows));
  const uint32_t trig_addr = wave_addr + enc_perm_bytes<D>(STAGE);
  // permutation: this vector's LDS row and the lane's 32 gather addresses
  const uint32_t row_addr = wave_addr + (uint32_t)(q * enc_row<D>());
  uint32_t gaddr[PERM_ANY ? 32 : 1];
  if constexpr (PERM_ANY) {
    if (PERM) {
      // the lane's 32 offsets (64 bytes of the block's table), two per word
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4_t w = lds_ld4(lds_addr(s_goff) + 64u * l + 16u * k);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gaddr[8 * k + 2 * e] = row_addr + (ws[e] & 0xffffu);
          gaddr[8 * k + 2 * e + 1] = row_addr + (ws[e] >> 16);
        }
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) asm volatile("" : "+v"(gaddr[i]));  // keep the sums (not offsets re-added per item)
    }
  }

  uint32_t swz[8];  // byte offset of the lane's 16-byte piece k in its row or table slice
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    swz[k] = 16u * (uint32_t)((k + l) & 7);
    asm volatile("" : "+v"(swz[k]));
  }
  const float norm_c = (ROT == ROT_FWHT) ? (float)(1.0 / __builtin_sqrt((double)D)) : 1.0f;
  const float sgn = (ROT == ROT_FWHT) ? lane_sign(l) : 1.0f;
  const float A = sgn * norm_c;  // true rotated coefficient = A * (value held by this lane)
  const float m1 = (l & 1) ? -1.0f : 1.0f, m2 = (l & 2) ? -1.0f : 1.0f, m4 = (l & 4) ? -1.0f : 1.0f;
  const int gb = (GBT > 0) ? GBT : a.group_log2;
  const int LB = (QUANT == Q_MINMAX) ? gb - 5 : 0;  // lane bits inside a group (G >= 32)
  const int64_t ngroups = (QUANT == Q_MINMAX) ? (D >> gb) : 0;

  // lane state of the current tile; the wave's RoPE table holds cos/sin of (token, pair)
  // for the tokens t0 .. t0 + ntok - 1 the tile spans
  LaneTile cur = lane_tile<VPW>(a, wk.tile, q);
  auto set_trig = [&](const LaneTile& lt) __attribute__((always_inline)) {
    if constexpr (ROPE_ANY) {
      if (ROPE) {
        const uint32_t last = (uint32_t)(min(lt.tile * VPW + VPW, ncols) - 1);  // < 2^31
        const int ntok = (int)(fdiv(last, a.div_heads) - (uint32_t)lt.t0) + 1;
        const int64_t p0 = (AP ? prow : a.pos_offset) + lt.t0;
        wave_lds_sync();  // the previous tile's table has been read
        for (int m = lane; m < ntok * (D / 2); m += 64) {
          const int tok = m / (D / 2), i = m % (D / 2);
          float c, sn;
          rope_cos_sin(p0 + tok, s_theta[i], &c, &sn);
          u32x2_t w = {__float_as_uint(c), __float_as_uint(sn)};
          const int li = i >> 4, pi = i & 15;
          const uint32_t ta = trig_addr + (uint32_t)(tok * trig_row<D>() + li * kTrigLane + 16 * (((pi >> 1) + li) & 7) + 8 * (pi & 1));
          *(__attribute__((address_space(3))) u32x2_t*)(uintptr_t)ta = w;
        }
        wave_lds_sync();
      }
    }
  };
  // input of an item: from the tile's first token of the row (wave-uniform) up to the
  // row's last element; lanes of columns past the end start beyond it.  The lane's offset
  // fits in 31 bits (checked on the host).
  auto in_buf = [&](const LaneTile& lt, int64_t row, bool on) __attribute__((always_inline)) -> buf_t {
    const int64_t span = ((a.tokens - 1 - lt.t0) * a.st + (a.heads - 1) * a.sh + D) * ES;
    return make_buf(reinterpret_cast<const char*>(a.x) + (on ? (row * a.sr + lt.t0 * a.st) * ES : 0),
                    on ? span : 0);
  };
  auto in_off = [&](const LaneTile& lt) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)(((int64_t)lt.dtok * a.st + (int64_t)lt.h * a.sh + 32 * l) * ES);
  };

  // Every lane computes; the stores of lanes past the end of the tensor are dropped.
  auto process = [&](const RawRow<DT>& raw, const LaneTile& lt, int64_t row) __attribute__((always_inline)) {
    int64_t vec0 = row * ncols + lt.tile * VPW;                // first vector of the item in the planes
    int64_t nvalid = min(ncols - lt.tile * VPW, (int64_t)VPW);  // vectors of the item that exist
    if constexpr (AP) {
      // the row's slot in the cache; a position outside the cache's slots writes nothing
      const int64_t slot = prow - a.pos_offset;
      const bool in = slot >= 0 && slot < a.cap;
      vec0 = in ? (row * a.cap + slot) * a.heads + lt.tile * VPW : 0;
      nvalid = in ? nvalid : 0;
      if (prow < a.n_sink) {
        // a sink position (wave-uniform: the item is one row at one position): fp16 of the
        // post-RoPE vector into the sink plane, zeros into the vector's other slots
        float v[32];
        widen_row<DT>(raw, v);
        if constexpr (ROPE_ANY) {
          if (ROPE) {
            const uint32_t tp0 = trig_addr + (uint32_t)(lt.dtok * trig_row<D>() + kTrigLane * l);
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
              for (int hh = 0; hh < 2; ++hh) {
                const u32x4_t cs = lds_ld4(tp0 + swz[2 * c + hh]);
                float* w = v + 8 * c + 4 * hh;
                const float x0 = w[0], x1 = w[1], x2 = w[2], x3 = w[3];
                w[0] = __builtin_fmaf(x0, __uint_as_float(cs.x), -x1 * __uint_as_float(cs.y));
                w[1] = __builtin_fmaf(x0, __uint_as_float(cs.y), x1 * __uint_as_float(cs.x));
                w[2] = __builtin_fmaf(x2, __uint_as_float(cs.z), -x3 * __uint_as_float(cs.w));
                w[3] = __builtin_fmaf(x2, __uint_as_float(cs.w), x3 * __uint_as_float(cs.z));
              }
          }
        }
        const buf_t sb = make_buf_item(a.sink + ((row * a.n_sink + prow) * a.heads + lt.tile * VPW) * D,
                                       (uint32_t)(nvalid * D * 2));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const u32x4_t w = {pack_f16x2(v[8 * k + 0], v[8 * k + 1]), pack_f16x2(v[8 * k + 2], v[8 * k + 3]),
                             pack_f16x2(v[8 * k + 4], v[8 * k + 5]), pack_f16x2(v[8 * k + 6], v[8 * k + 7])};
          __builtin_amdgcn_raw_buffer_store_b128(w, sb, (uint32_t)((q * D + 32 * l) * 2 + 16 * k), 0, 0);
        }
        LaneCodes<BITS> zc;
#pragma unroll
        for (int w = 0; w < BITS; ++w) zc.w[w] = 0u;
        store_lane_codes<BITS>(make_buf_item(a.codes + vec0 * CB, (uint32_t)(CB * nvalid)),
                               (uint32_t)(q * CB + l * (4 * BITS)), zc);
        if constexpr (QUANT == Q_MINMAX) {
          const uint32_t gbytes = (uint32_t)(2 * nvalid * ngroups);
          const uint32_t go = 2u * (uint32_t)(q * ngroups + (l >> LB));
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, make_buf_item(a.scale + vec0 * ngroups, gbytes), go, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, make_buf_item(a.zero + vec0 * ngroups, gbytes), go, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(0u, make_buf_item(a.norm + vec0, (uint32_t)(4 * nvalid)),
                                                4u * (uint32_t)q, 0, 0);
          if (a.dyn && l == 0) {
            constexpr int EB = D / 128;
            const buf_t eb = make_buf_item(a.extra + vec0 * EB, (uint32_t)(EB * nvalid));
            if constexpr (EB == 1) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)0, eb, (uint32_t)q, 0, 0);
            else __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, eb, 2u * (uint32_t)q, 0, 0);
          }
        }
        return;
      }
    }
    float v[32];
    // RoPE of the 4 channel pairs of 8 consecutive slots 8c .. 8c + 7
    auto rope8 = [&](float* u, int c) __attribute__((always_inline)) {
      const uint32_t tp = trig_addr + (uint32_t)(lt.dtok * trig_row<D>() + kTrigLane * l);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4_t cs = lds_ld4(tp + swz[2 * c + h]);
        const float c0 = __uint_as_float(cs.x), s0 = __uint_as_float(cs.y);
        const float c1 = __uint_as_float(cs.z), s1 = __uint_as_float(cs.w);
        float* w = u + 4 * h;
        const float x0 = w[0], x1 = w[1], x2 = w[2], x3 = w[3];
        w[0] = __builtin_fmaf(x0, c0, -x1 * s0);
        w[1] = __builtin_fmaf(x0, s0, x1 * c0);
        w[2] = __builtin_fmaf(x2, c1, -x3 * s1);
        w[3] = __builtin_fmaf(x2, s1, x3 * c1);
      }
    };
    bool staged = false;
    if constexpr (PERM_ANY) {
      if (PERM) {
        // widen (and rotate by RoPE) 8 slots at a time straight into the vector's staging
        // row in natural order, then gather u'[j] = u[perm[j]]
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float t[8];
          widen_chunk<DT>(raw, c, t);
          if constexpr (ROPE_ANY) {
            if (ROPE) rope8(t, c);
          }
          const u32x4_t w0 = {__float_as_uint(t[0]), __float_as_uint(t[1]), __float_as_uint(t[2]), __float_as_uint(t[3])};
          const u32x4_t w1 = {__float_as_uint(t[4]), __float_as_uint(t[5]), __float_as_uint(t[6]), __float_as_uint(t[7])};
          lds_st4(row_addr + (uint32_t)enc_pitch<D>() * l + swz[2 * c], w0);
          lds_st4(row_addr + (uint32_t)enc_pitch<D>() * l + swz[2 * c + 1], w1);
        }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = lds_ld(gaddr[i]);
        wave_lds_sync();
        staged = true;
      }
    }
    if (!staged) {
      if constexpr (FUSED) {
        widen_row_h4<DT>(raw, v);  // 16-bit input with the first two butterfly stages
      } else {
        widen_row<DT>(raw, v);
        if constexpr (ROPE_ANY) {
          if (ROPE) {
#pragma unroll
            for (int c = 0; c < 4; ++c) rope8(v + 8 * c, c);
          }
        }
      }
    }
    if constexpr (QUANT == Q_LLOYD) {
      // |u| (the permutation does not change it)
      const float rho = norm_separate<LV>(v);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(rho), make_buf_item(a.norm + vec0, (uint32_t)(4 * nvalid)),
                                            4u * (uint32_t)q, 0, 0);
    }
    if constexpr (ROT == ROT_FWHT) {
      fwht_lane<LV, FUSED ? 2 : 0>(v, m1, m2, m4);
    } else if constexpr (ROT == ROT_ROTOR) {
      rotor_lane<D, false>(v, row_addr, l, lds_addr(s_rtab));
    } else if constexpr (ROT == ROT_SO4) {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const float* m = &s_mat[16 * (8 * l + b)];
        float* u = v + 4 * b;
        const float u0 = u[0], u1 = u[1], u2 = u[2], u3 = u[3];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          u[i] = __builtin_fmaf(m[4 * i], u0,
                 __builtin_fmaf(m[4 * i + 1], u1, __builtin_fmaf(m[4 * i + 2], u2, m[4 * i + 3] * u3)));
      }
    }
    LaneCodes<BITS> cw;
    if constexpr (QUANT == Q_MINMAX) {
      uint32_t zb, sb;
      minmax_codes_lane<BITS, ROT == ROT_NONE>(v, A, LB, zb, sb, cw);
      {
        // every lane of a group holds the same values and stores them
        const uint32_t go = 2u * (uint32_t)(q * ngroups + (l >> LB));
        const uint32_t gbytes = (uint32_t)(2 * nvalid * ngroups);
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)sb, make_buf_item(a.scale + vec0 * ngroups, gbytes), go, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)zb, make_buf_item(a.zero + vec0 * ngroups, gbytes), go, 0, 0);
      }
    } else {
      // Lloyd-Max: q = #{k : z > tau_k}
      constexpr int NT = (1 << BITS) - 1;
      float tau[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) tau[i] = 0.5f * (a.codebook[i] + a.codebook[i + 1]);
      if (!a.dyn) {
        lloyd_codes_lane<BITS>(v, A, tau, cw);
      } else {
#pragma unroll
        for (int w = 0; w < BITS; ++w) cw.w[w] = 0u;
        // dynamic codebook: channel j compares z_j / scale_j against the N(0,1) midpoints; a wide
        // channel against the 2^(b+1)-level codebook's, its top code bit going to the extra plane
        constexpr int NTW = (2 << BITS) - 1;
        float tw[NTW];
#pragma unroll
        for (int i = 0; i < NTW; ++i) tw[i] = 0.5f * (a.codebook_wide[i] + a.codebook_wide[i + 1]);
        uint32_t ex = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int j = 32 * l + i;
          const float t = (v[i] * A) * s_cinv[j];
          const uint32_t rk = s_rank[j];
          uint32_t c = 0;
          if (rk != 0xffu) {
#pragma unroll
            for (int k = 0; k < NTW; ++k) c += (t > tw[k]) ? 1u : 0u;
            ex |= (c >> BITS) << rk;
            c &= (1u << BITS) - 1u;
          } else {
#pragma unroll
            for (int k = 0; k < NT; ++k) c += (t > tau[k]) ? 1u : 0u;
          }
          const int bit = BITS * i, w = bit >> 5, sh = bit & 31;
          cw.w[w] |= c << sh;
          if (BITS == 3 && sh > 29) cw.w[w + 1] |= c >> (32 - sh);
        }
        ex = vec_or<LV>(ex);
        constexpr int EB = D / 128;  // extra bytes per vector
        const buf_t eb = make_buf_item(a.extra + vec0 * EB, (uint32_t)(EB * nvalid));
        if (l == 0) {
          if constexpr (EB == 1) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)ex, eb, (uint32_t)q, 0, 0);
          else __builtin_amdgcn_raw_buffer_store_b16((uint16_t)ex, eb, 2u * (uint32_t)q, 0, 0);
        }
      }
    }
    store_lane_codes<BITS>(make_buf_item(a.codes + vec0 * CB, (uint32_t)(CB * nvalid)),
                           (uint32_t)(q * CB + l * (4 * BITS)), cw);
  };

  // the task's items, with the next item's loads in flight
  RawRow<DT> ra, rb;
  load_row<DT>(ra, in_buf(cur, wk.r, true), in_off(cur));
  {
    // the stores of an item, on size-0 descriptors (nothing is written): the loop is then
    // entered with the same outstanding memory instructions on every path, and the
    // compiler's wait for an item's loads does not also wait for earlier stores
    const buf_t nb = make_buf_item(a.codes, 0);
    if constexpr (QUANT == Q_MINMAX) {
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, nb, 0, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, nb, 16, 0, 0);  // distinct, so none is merged
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(0u, nb, 0, 0, 0);
    }
    LaneCodes<BITS> z{};
    store_lane_codes<BITS>(nb, 32, z);
  }
  set_trig(cur);  // while the first loads are in flight
  LaneTile nxt = cur;
  auto step = [&](RawRow<DT>& now, RawRow<DT>& later) __attribute__((always_inline)) -> bool {
    Walk nw = wk;
    const bool more = walk_next_rows(nw);
    if (more && nw.tile != cur.tile) nxt = lane_tile<VPW>(a, nw.tile, q);
    // the next item's loads go out before this item's work (after the last item they
    // fall outside the buffer and move nothing)
    load_row<DT>(later, in_buf(nxt, nw.r, more), in_off(nxt));
    __builtin_amdgcn_sched_barrier(0);
    process(now, cur, wk.r);
    if (!more) return false;
    wk = nw;
    if (nxt.tile != cur.tile) {
      cur = nxt;
      set_trig(cur);
    }
    return true;
  };
  while (step(ra, rb) && step(rb, ra)) {
  }
}

// ---------------------------------------------------------------------------
// DECODE
// ---------------------------------------------------------------------------
// PT: permutation off (0), on (1) or read from the arguments (-1).
// FWHT + min-max runs the in-lane Walsh-Hadamard stages on the integer codes (packed
// 16-bit pairs, exact), then scales once per element and finishes the lane stages in
// float; other rotations and quantizers dequantize first and rotate in float.
template <int ODT, int D, int BITS, int ROT, int QUANT, int PT>
__global__ void __launch_bounds__(64 * kWavesPerBlock) decode_kernel(const CodecArgs a) {
  using G = Geo<D>;
  constexpr int LV = G::LV, VPW = G::VPW;
  constexpr bool PERM_ANY = PT != 0;
  constexpr bool INTPATH = (ROT == ROT_FWHT) && (QUANT == Q_MINMAX);
  const bool PERM = (PT < 0) ? (a.use_perm != 0) : (PT == 1);
  extern __shared__ float s_stage[];
  __shared__ float s_mat[ROT == ROT_SO4 ? (D / 4) * 16 : 1];
  __shared__ float s_cb[kMaxCodebook];
  // permutation: byte offset of channel perm[j] in a staging row (output type), for the scatter
  __shared__ __attribute__((aligned(16))) uint16_t s_soff[PERM_ANY ? D : 8];
  __shared__ __attribute__((aligned(16))) float s_rtab[ROT == ROT_ROTOR ? (D / 3 + 1) * 12 : 4];
  // dynamic codebook: the wide codebook, each rotated channel's scale and wide-channel rank
  __shared__ float s_cbw[QUANT == Q_LLOYD ? 2 * kMaxCodebook : 1];
  __shared__ float s_csc[QUANT == Q_LLOYD ? D : 1];
  __shared__ uint8_t s_rank[QUANT == Q_LLOYD ? D : 1];

  const int tid = threadIdx.x;
  constexpr int OES = (ODT == DT_F32) ? 4 : 2;
  if constexpr (ROT == ROT_SO4) {
    for (int b = tid; b < D / 4; b += blockDim.x) build_so4(&a.quat[8 * b], &s_mat[16 * b]);
  }
  if constexpr (PERM_ANY) {
    if (PERM)
      for (int j = tid; j < D; j += blockDim.x) s_soff[j] = (uint16_t)(OES * (uint32_t)a.perm[j]);
  }
  if constexpr (ROT == ROT_ROTOR) build_rotor_table<D>(a.quat, s_rtab);
  if constexpr (QUANT == Q_LLOYD) {
    if (tid < (1 << BITS)) s_cb[tid] = a.codebook[tid];
    if (a.dyn) {
      if (tid < (2 << BITS)) s_cbw[tid] = a.codebook_wide[tid];
      for (int j = tid; j < D; j += blockDim.x) {
        s_csc[j] = a.chan_scale[j];
        s_rank[j] = a.wide_rank[j];
      }
    }
  }
  // block-shared parameters ready; the barrier also starts the block's four waves (adjacent
  // tiles) together, which measured about 2 % faster even where there are no parameters
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const uint32_t wid = blockIdx.x * kWavesPerBlock + (uint32_t)wave;
  Walk wk;
  if (!walk_first_tiles(a, wid, wk)) return;  // wave-uniform; no barrier follows

  const int q = lane / LV, l = lane % LV;
  const int64_t ncols = a.tokens * a.heads;
  constexpr int CB = D * BITS / 8;
  const float norm_c = (ROT == ROT_FWHT) ? (float)(1.0 / __builtin_sqrt((double)D)) : 1.0f;
  const float sgn = (ROT == ROT_FWHT) ? lane_sign(l) : 1.0f;
  const int gb = a.group_log2;
  const int LB = (QUANT == Q_MINMAX) ? gb - 5 : 0;
  const int64_t ngroups = (QUANT == Q_MINMAX) ? (D >> gb) : 0;

  // staging rows: vector q's row; in the permuted case the lane scatters its 32 floats
  // to out[perm[j]], otherwise it writes its 32 outputs (in the output type) in order
  constexpr int ROWB = dec_row_bytes<D, ODT>();
  // the rotor's float rows follow the wave's output rows
  constexpr int RROW = D * 4 + 16, RBYTES = (ROT == ROT_ROTOR) ? Geo<D>::VPW * RROW : 0;
  const uint32_t wave_addr = lds_addr(s_stage) + (uint32_t)(wave * (Geo<D>::VPW * ROWB + RBYTES));
  const uint32_t rrow_addr = wave_addr + (uint32_t)(Geo<D>::VPW * ROWB + q * RROW);
  const uint32_t row_addr = wave_addr + (uint32_t)(q * ROWB);
  uint32_t saddr[PERM_ANY ? 32 : 1];
  if constexpr (PERM_ANY) {
    if (PERM) {
      // the lane's 32 offsets (64 bytes of the block's table), two per word
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4_t w = lds_ld4(lds_addr(s_soff) + 64u * l + 16u * k);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          saddr[8 * k + 2 * e] = row_addr + (ws[e] & 0xffffu);
          saddr[8 * k + 2 * e + 1] = row_addr + (ws[e] >> 16);
        }
      }
    }
  }

  struct Packed {
    LaneCodes<BITS> c;
    uint32_t sc, zr;  // fp16 bits of scale and zero (min-max), combined only where used,
                      // so that nothing waits for the prefetch before the current item
    float rho;    // Lloyd-Max
    uint32_t ex;  // dynamic codebook: the vector's extra bits
  };
  // the packed planes of item (tile, row); with on == false (wave-uniform) nothing is read
  auto fetch = [&](Packed& pk, const LaneTile& lt, int64_t row, bool on) __attribute__((always_inline)) {
    const int64_t vec0 = on ? row * ncols + lt.tile * VPW : 0;  // first vector of the item
    const int64_t nvalid = on ? min(ncols - lt.tile * VPW, (int64_t)VPW) : 0;  // its vectors that exist
    load_lane_codes<BITS>(make_buf(a.codes + vec0 * CB, CB * nvalid), (uint32_t)(q * CB + l * (4 * BITS)), pk.c);
    if constexpr (QUANT == Q_MINMAX) {
      const uint32_t go = 2u * (uint32_t)(q * ngroups + (l >> LB));
      const int64_t gbytes = 2 * nvalid * ngroups;
      // temporal: lanes share the lines of these 2-byte values (with the non-temporal hint
      // the decoders fetched 16 % more than the planes hold)
      const uint16_t sc = __builtin_amdgcn_raw_buffer_load_b16(make_buf(a.scale + vec0 * ngroups, gbytes), go, 0, 0);
      const uint16_t zr = __builtin_amdgcn_raw_buffer_load_b16(make_buf(a.zero + vec0 * ngroups, gbytes), go, 0, 0);
      pk.sc = sc;
      pk.zr = zr;
    } else {
      pk.rho = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(make_buf(a.norm + vec0, 4 * nvalid), 4u * (uint32_t)q, 0, kNT));
      pk.ex = 0u;
      if (a.dyn) {
        constexpr int EB = D / 128;
        const buf_t eb = make_buf(a.extra + vec0 * EB, EB * nvalid);
        if constexpr (EB == 1) pk.ex = __builtin_amdgcn_raw_buffer_load_b8(eb, (uint32_t)q, 0, 0);
        else pk.ex = __builtin_amdgcn_raw_buffer_load_b16(eb, 2u * (uint32_t)q, 0, 0);
      }
    }
  };

  // a lane's 32 output values, true coefficients in natural slot order
  auto reconstruct = [&](const Packed& pk, float* v) __attribute__((always_inline)) {
    if constexpr (INTPATH) {
      // packed pairs: word s holds codes (s, s + 16) as 16-bit integers
      uint32_t w[16];
      if constexpr (BITS == 2) {
        // bytes of c.w[0] hold codes 0-3, 4-7, 8-11, 12-15; c.w[1] codes 16-31
        const uint32_t plo = __builtin_amdgcn_perm(pk.c.w[1], pk.c.w[0], 0x05040100u);  // codes 0-7 | 16-23
        const uint32_t phi = __builtin_amdgcn_perm(pk.c.w[1], pk.c.w[0], 0x07060302u);  // codes 8-15 | 24-31
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          w[s] = (plo >> (2 * s)) & 0x00030003u;
          w[s + 8] = (phi >> (2 * s)) & 0x00030003u;
        }
      } else if constexpr (BITS == 4) {
        // c.w[0]: codes 0-7, c.w[1]: 8-15, c.w[2]: 16-23, c.w[3]: 24-31
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t plo = __builtin_amdgcn_perm(pk.c.w[2 + h], pk.c.w[h], 0x05040100u);
          const uint32_t phi = __builtin_amdgcn_perm(pk.c.w[2 + h], pk.c.w[h], 0x07060302u);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            w[8 * h + s] = (plo >> (4 * s)) & 0x000F000Fu;
            w[8 * h + s + 4] = (phi >> (4 * s)) & 0x000F000Fu;
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < 16; ++s) w[s] = code_at<3>(pk.c, s) | (code_at<3>(pk.c, s + 16) << 16);
      }
      // Walsh-Hadamard over slot bits 0..3 between words, exact in 16-bit lanes
#pragma unroll
      for (int hb = 1; hb < 16; hb <<= 1) {
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          if (s & hb) continue;
          const i16x2_t x = __builtin_bit_cast(i16x2_t, w[s]), y = __builtin_bit_cast(i16x2_t, w[s + hb]);
          w[s] = __builtin_bit_cast(uint32_t, (i16x2_t)(x + y));
          w[s + hb] = __builtin_bit_cast(uint32_t, (i16x2_t)(x - y));
        }
      }
      // slot bit 4, inside each word: (lo, hi) -> (lo + hi, lo - hi), one v_pk_mad_u16
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const i16x2_t x = __builtin_bit_cast(i16x2_t, w[s]);
        const i16x2_t pm = {1, -1};
        w[s] = __builtin_bit_cast(uint32_t, (i16x2_t)(x.yy * pm + x.xx));
      }
      // value = zero + q * scale per group: H_32 of (zero * ones) puts 32 * zero on slot 0.
      // The lane's inputs to the lane stages carry (-1)^popcount(l) so that the stages
      // below (m = +1 on a set bit) yield the true coefficients, times 1/sqrt(D).
      const float sc = f16_value(pk.sc), z = f16_value(pk.zr);
      const float S = sgn * norm_c * sc;
      const float Z0 = sgn * norm_c * 32.0f * z;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        v[s] = (float)(short)(w[s] & 0xffffu) * S;
        v[s + 16] = (float)((int)w[s] >> 16) * S;
      }
      v[0] = __builtin_fmaf((float)(short)(w[0] & 0xffffu), S, Z0);
      const float p1 = (l & 1) ? 1.0f : -1.0f, p2 = (l & 2) ? 1.0f : -1.0f, p4 = (l & 4) ? 1.0f : -1.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) fmac_x1(v + 8 * k, p1);
#pragma unroll
      for (int k = 0; k < 4; ++k) fmac_x2(v + 8 * k, p2);
      if constexpr (LV == 8) {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(swz_x4(v[i]), p4, v[i]);
      }
    } else {
      if constexpr (QUANT == Q_MINMAX) {
        const float sc = f16_value(pk.sc), z = f16_value(pk.zr);
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf((float)code_at<BITS>(pk.c, i), sc, z);
      } else if (!a.dyn) {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = s_cb[code_at<BITS>(pk.c, i)];
      } else {
        // dynamic codebook: scale_j times the level of the channel's own codebook
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int j = 32 * l + i;
          const uint32_t c = code_at<BITS>(pk.c, i), rk = s_rank[j];
          const float lev = (rk != 0xffu) ? s_cbw[c | (((pk.ex >> (rk & 31u)) & 1u) << BITS)] : s_cb[c];
          v[i] = lev * s_csc[j];
        }
      }
      float outscale = 1.0f;
      if constexpr (ROT == ROT_FWHT) {
        const float m1 = (l & 1) ? -1.0f : 1.0f, m2 = (l & 2) ? -1.0f : 1.0f, m4 = (l & 4) ? -1.0f : 1.0f;
        fwht_lane<LV>(v, m1, m2, m4);
        outscale = sgn * norm_c;
      } else if constexpr (ROT == ROT_ROTOR) {
        rotor_lane<D, true>(v, rrow_addr, l, lds_addr(s_rtab));
      } else if constexpr (ROT == ROT_SO4) {
        // inverse: M^T z (M orthogonal for unit quaternions)
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const float* m = &s_mat[16 * (8 * l + b)];
          float* u = v + 4 * b;
          const float u0 = u[0], u1 = u[1], u2 = u[2], u3 = u[3];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            u[i] = __builtin_fmaf(m[i], u0, __builtin_fmaf(m[4 + i], u1, __builtin_fmaf(m[8 + i], u2, m[12 + i] * u3)));
        }
      }
      if constexpr (QUANT == Q_LLOYD) outscale *= pk.rho;
      if (ROT == ROT_FWHT || QUANT == Q_LLOYD) {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] *= outscale;
      }
    }
  };

  // One item: every lane puts its 32 outputs into its vector's staging row, then the wave
  // stores the tile's output as contiguous 1 KiB runs (16 bytes per lane); the runs of
  // vectors past the end of the tensor fall outside the store descriptor.
  constexpr int ITEM_BYTES = VPW * D * OES;   // contiguous output bytes of a full tile
  constexpr int NCHUNK = ITEM_BYTES / 1024;
  constexpr int VBYTES = D * OES;             // output bytes per vector
  auto process = [&](const Packed& pk, const LaneTile& lt, int64_t row) __attribute__((always_inline)) {
    {
      float v[32];
      reconstruct(pk, v);
      if constexpr (PERM_ANY) {
        if (PERM) {
          // scatter out[perm[j]] = v[j] in the output type
          if constexpr (ODT == DT_F32) {
#pragma unroll
            for (int i = 0; i < 32; ++i) lds_st(saddr[i], v[i]);
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const uint32_t h2 = (ODT == DT_BF16) ? pack_bf16x2(v[2 * i], v[2 * i + 1]) : pack_f16x2(v[2 * i], v[2 * i + 1]);
              lds_st16(saddr[2 * i], (uint16_t)h2);
              lds_st16(saddr[2 * i + 1], (uint16_t)(h2 >> 16));
            }
          }
        }
      }
      if (!(PERM_ANY && PERM)) {
        // the lane's 32 outputs in the output type, in order
        if constexpr (ODT == DT_F32) {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            u32x4_t w = {__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]), __float_as_uint(v[4 * k + 2]),
                         __float_as_uint(v[4 * k + 3])};
            lds_st4(row_addr + 128u * l + 16u * k, w);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            u32x4_t w;
            if constexpr (ODT == DT_BF16) {
              w.x = pack_bf16x2(v[8 * k + 0], v[8 * k + 1]);
              w.y = pack_bf16x2(v[8 * k + 2], v[8 * k + 3]);
              w.z = pack_bf16x2(v[8 * k + 4], v[8 * k + 5]);
              w.w = pack_bf16x2(v[8 * k + 6], v[8 * k + 7]);
            } else {
              w.x = pack_f16x2(v[8 * k + 0], v[8 * k + 1]);
              w.y = pack_f16x2(v[8 * k + 2], v[8 * k + 3]);
              w.z = pack_f16x2(v[8 * k + 4], v[8 * k + 5]);
              w.w = pack_f16x2(v[8 * k + 6], v[8 * k + 7]);
            }
            lds_st4(row_addr + 64u * l + 16u * k, w);
          }
        }
      }
    }
    wave_lds_sync();
    // contiguous stores: chunk c, lane L covers output bytes c*1024 + L*16 of the tile
    const int64_t nvalid = min(ncols - lt.tile * VPW, (int64_t)VPW);  // vectors of this tile that exist
    const buf_t yb = make_buf(reinterpret_cast<char*>(a.y) + (row * ncols + lt.tile * VPW) * (int64_t)VBYTES,
                              nvalid * VBYTES);
#pragma unroll
    for (int c = 0; c < NCHUNK; ++c) {
      const int off = c * 1024 + lane * 16;
      const int vq = off / VBYTES, inner = off % VBYTES;
      {
        // rows hold the vectors in the output type, in channel order
        const u32x4_t w = lds_ld4(wave_addr + (uint32_t)(vq * ROWB + inner));
        __builtin_amdgcn_raw_buffer_store_b128(w, yb, (uint32_t)off, 0, kNT | kSC1);
      }
    }
    wave_lds_sync();
  };

  // the task's items, with the next item's packed planes in flight
  LaneTile cur = lane_tile<VPW>(a, wk.tile, q);
  Packed pa, pb;
  fetch(pa, cur, wk.r, true);
  // the stores of an item, on a size-0 descriptor (nothing is written): the loop is then
  // entered with the same outstanding memory instructions on every path, and the
  // compiler's wait for an item's loads does not also wait for earlier stores
#pragma unroll
  for (int c = 0; c < NCHUNK; ++c)  // distinct offsets, so none is merged
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{0u, 0u, 0u, 0u}, make_buf(a.y, 0), 16u * c, 0, 0);
  LaneTile nxt = cur;
  auto step = [&](Packed& now, Packed& later) __attribute__((always_inline)) -> bool {
    Walk nw = wk;
    const bool more = walk_next_tiles(nw);
    if (more && nw.tile != cur.tile) nxt = lane_tile<VPW>(a, nw.tile, q);
    fetch(later, nxt, nw.r, more);  // in flight during this item's work
    __builtin_amdgcn_sched_barrier(0);
    process(now, cur, wk.r);
    if (!more) return false;
    wk = nw;
    cur = nxt;
    return true;
  };
  while (step(pa, pb) && step(pb, pa)) {
  }
}

// ---------------------------------------------------------------------------
// ATTENTION SINKS
// ---------------------------------------------------------------------------
// Positions p < n_sink are kept as fp16 of the post-RoPE, unrotated vector.  The main
// kernels treat every vector alike; these small kernels run after them on the same
// stream and cover only the sink positions of the call: the encoder's writes the sink
// plane and zeroes the vector's code, scale, zero and norm slots, the decoder's copies
// the sink plane to the output.  One sub-wavefront per vector, as in the main kernels.
__device__ __forceinline__ int64_t sink_tokens(const CodecArgs& a) {
  const int64_t n = (int64_t)a.n_sink - a.pos_offset;
  return n <= 0 ? 0 : (n < a.tokens ? n : a.tokens);
}

template <int DT, int D, int BITS, int QUANT>
__global__ void __launch_bounds__(64 * kWavesPerBlock) encode_sink_kernel(const CodecArgs a) {
  constexpr int LV = Geo<D>::LV;
  constexpr int ES = (DT == DT_F32) ? 4 : 2;
  constexpr int CB = D * BITS / 8;
  const int64_t nt = sink_tokens(a);
  const int64_t g = (int64_t)blockIdx.x * (blockDim.x / LV) + threadIdx.x / LV;  // (row, token, head)
  const int l = threadIdx.x % LV;
  if (g >= a.rows * nt * a.heads) return;
  const int64_t h = g % a.heads, rt = g / a.heads, t = rt % nt, r = rt / nt;
  const int64_t pos = a.pos_offset + t;
  RawRow<DT> raw;
  load_row<DT>(raw, reinterpret_cast<const char*>(a.x) + (r * a.sr + t * a.st + h * a.sh + 32 * l) * ES);
  float v[32];
  widen_row<DT>(raw, v);
  if (a.rope) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int i = 16 * l + m;  // pair index
      const double theta = exp2(-(2.0 * (double)i / (double)D) * a.rope_log2_base);
      float c, sn;
      rope_cos_sin(pos, theta, &c, &sn);
      const float x0 = v[2 * m], x1 = v[2 * m + 1];
      v[2 * m] = __builtin_fmaf(x0, c, -x1 * sn);
      v[2 * m + 1] = __builtin_fmaf(x0, sn, x1 * c);
    }
  }
  const int64_t srow = (r * a.n_sink + pos) * a.heads + h;
  u32x4_t* sp = reinterpret_cast<u32x4_t*>(a.sink + srow * D + 32 * l);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    u32x4_t w;
    w.x = pack_f16x2(v[8 * k + 0], v[8 * k + 1]);
    w.y = pack_f16x2(v[8 * k + 2], v[8 * k + 3]);
    w.z = pack_f16x2(v[8 * k + 4], v[8 * k + 5]);
    w.w = pack_f16x2(v[8 * k + 6], v[8 * k + 7]);
    sp[k] = w;
  }
  const int64_t vec = (r * a.tokens + t) * a.heads + h;
  LaneCodes<BITS> zc;
#pragma unroll
  for (int w = 0; w < BITS; ++w) zc.w[w] = 0u;
  store_lane_codes<BITS>(a.codes + vec * CB + l * (4 * BITS), zc);
  if constexpr (QUANT == Q_MINMAX) {
    const int LB = a.group_log2 - 5;
    const int64_t ngroups = D >> a.group_log2;
    if ((l & ((1 << LB) - 1)) == 0) {
      a.scale[vec * ngroups + (l >> LB)] = 0;
      a.zero[vec * ngroups + (l >> LB)] = 0;
    }
  } else {
    if (l == 0) a.norm[vec] = 0.0f;
    if (a.dyn && l == 0)
      for (int e = 0; e < D / 128; ++e) a.extra[vec * (D / 128) + e] = 0;
  }
}

template <int ODT, int D>
__global__ void __launch_bounds__(64 * kWavesPerBlock) decode_sink_kernel(const CodecArgs a) {
  constexpr int LV = Geo<D>::LV;
  const int64_t nt = sink_tokens(a);
  const int64_t g = (int64_t)blockIdx.x * (blockDim.x / LV) + threadIdx.x / LV;
  const int l = threadIdx.x % LV;
  if (g >= a.rows * nt * a.heads) return;
  const int64_t h = g % a.heads, rt = g / a.heads, t = rt % nt, r = rt / nt;
  const int64_t pos = a.pos_offset + t;
  const int64_t srow = (r * a.n_sink + pos) * a.heads + h;
  const u32x4_t* sp = reinterpret_cast<const u32x4_t*>(a.sink + srow * D + 32 * l);
  const int64_t vec = (r * a.tokens + t) * a.heads + h;
  if constexpr (ODT == DT_F16) {
    u32x4_t* yp = reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(a.y) + vec * D + 32 * l);
#pragma unroll
    for (int k = 0; k < 4; ++k) yp[k] = sp[k];
  } else {
    float v[32];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4_t w = sp[k];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * k + 2 * i] = f16_value(ws[i] & 0xffffu);
        v[8 * k + 2 * i + 1] = f16_value(ws[i] >> 16);
      }
    }
    if constexpr (ODT == DT_F32) {
      u32x4_t* yp = reinterpret_cast<u32x4_t*>(reinterpret_cast<float*>(a.y) + vec * D + 32 * l);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        u32x4_t w = {__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]), __float_as_uint(v[4 * k + 2]),
                     __float_as_uint(v[4 * k + 3])};
        yp[k] = w;
      }
    } else {
      u32x4_t* yp = reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(a.y) + vec * D + 32 * l);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        u32x4_t w;
        w.x = pack_bf16x2(v[8 * k + 0], v[8 * k + 1]);
        w.y = pack_bf16x2(v[8 * k + 2], v[8 * k + 3]);
        w.z = pack_bf16x2(v[8 * k + 4], v[8 * k + 5]);
        w.w = pack_bf16x2(v[8 * k + 6], v[8 * k + 7]);
        yp[k] = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// DENSE ROTATION (the baselines the IsoQuant page, section 1, compares against): z = M P u with
// an orthogonal d x d matrix, d = 128, on the fp32 matrix cores
// ---------------------------------------------------------------------------
// A block of 8 waves holds the matrix in LDS with the permutation folded in: the encoder's
// Q[i][perm[j]] = M[i][j] (Q u = M P u), the decoder's R[perm[j]][i] = M[i][j] (R z = P^T M^T z,
// the output in the original channel order).  128 rows of 528 bytes, loaded once per block;
// blocks then loop over items of 16 vectors, one wave per item.  Per item, every lane forms
// its 32 channels of one vector as the encoder (or decoder) does, stages them in the wave's 16
// LDS rows, and the wave computes Z^T = Q U^T with 256 v_mfma_f32_16x16x4f32: product (m, s)
// multiplies rows 16 m .. 16 m + 15 of Q (A operand, lane (n16, g): row 16 m + n16) with the
// 16 vectors (B operand, lane (n16, g): vector n16) over input channels 16 (s / 4) + 4 g + s % 4,
// so each lane reads 4 consecutive floats of a row for 4 products.  Lane (n16, g) then holds
// channels 16 m + 4 g .. + 3 of vector n16; they go back to LDS and are read in the codec's
// lane layout (lane l of a vector: channels 32 l .. 32 l + 31).  fp32 products and sums: the
// rotation is exact fp32 arithmetic up to the summation order.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kDenseWaves = 8;
constexpr int kDensePitch = 128 * 4 + 16;                            // bytes per LDS row
constexpr int kDenseLds = (128 + kDenseWaves * 16) * kDensePitch;  // 135168 bytes per block

// the wave's 16 staged rows (U) times the block's matrix rows: acc[m] = rows 16 m .. of Z^T
__device__ __forceinline__ void dense_product(uint32_t mat, uint32_t stage, int n16, int g, f32x4_t (&acc)[8]) {
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t col = 4u * (uint32_t)(16 * u + 4 * g);
    const u32x4_t b4 = lds_ld4(stage + (uint32_t)(n16 * kDensePitch) + col);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const u32x4_t a4 = lds_ld4(mat + (uint32_t)((16 * m + n16) * kDensePitch) + col);
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a4.x), __uint_as_float(b4.x), acc[m], 0, 0, 0);
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a4.y), __uint_as_float(b4.y), acc[m], 0, 0, 0);
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a4.z), __uint_as_float(b4.z), acc[m], 0, 0, 0);
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a4.w), __uint_as_float(b4.w), acc[m], 0, 0, 0);
    }
  }
}

// A lane's 32 values through the matrix: staged as vector q's row (channels 32 l ..), rotated
// by the wave, and read back in the same layout.
__device__ __forceinline__ void dense_rotate_lane(float* v, uint32_t mat, uint32_t stage, int q, int l, int n16,
                                                  int g) {
  const uint32_t row = stage + (uint32_t)(q * kDensePitch + 128 * l);
#pragma unroll
  for (int k = 0; k < 8; ++k)
    lds_st4(row + 16u * k, u32x4_t{__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]),
                                   __float_as_uint(v[4 * k + 2]), __float_as_uint(v[4 * k + 3])});
  wave_lds_sync();
  f32x4_t acc[8];
  dense_product(mat, stage, n16, g, acc);
  wave_lds_sync();  // every lane's reads of the staged rows are done
#pragma unroll
  for (int m = 0; m < 8; ++m)
    lds_st4(stage + (uint32_t)(n16 * kDensePitch) + 4u * (uint32_t)(16 * m + 4 * g),
            u32x4_t{__float_as_uint(acc[m][0]), __float_as_uint(acc[m][1]), __float_as_uint(acc[m][2]),
                    __float_as_uint(acc[m][3])});
  wave_lds_sync();
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const u32x4_t w = lds_ld4(row + 16u * k);
    v[4 * k] = __uint_as_float(w.x);
    v[4 * k + 1] = __uint_as_float(w.y);
    v[4 * k + 2] = __uint_as_float(w.z);
    v[4 * k + 3] = __uint_as_float(w.w);
  }
  wave_lds_sync();  // the rows are free for the next item
}

// The block's matrix into LDS with the permutation folded in: the encoder's Q[i][perm[j]] and
// the decoder's R[perm[j]][i] both hold M[i][j].
template <bool INVERSE>
__device__ __forceinline__ void dense_load_matrix(const CodecArgs& a, uint32_t mat) {
  for (int e = threadIdx.x; e < 128 * 128; e += blockDim.x) {
    const int i = e >> 7, j = e & 127;  // M[i][j]
    const int pj = a.use_perm ? a.perm[j] : j;
    const uint32_t off = INVERSE ? (uint32_t)(pj * kDensePitch + 4 * i) : (uint32_t)(i * kDensePitch + 4 * pj);
    lds_st(mat + off, a.rot_matrix[e]);
  }
}

template <int DT, int BITS, int QUANT>
__global__ void __launch_bounds__(64 * kDenseWaves) encode_dense_kernel(const CodecArgs a) {
  constexpr int D = 128, LV = 4, CB = D * BITS / 8;
  constexpr int ES = (DT == DT_F32) ? 4 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t s_dense[kDenseLds];
  __shared__ double s_theta[D / 2];
  const uint32_t mat = lds_addr(s_dense);
  dense_load_matrix<false>(a, mat);
  if (a.rope)
    for (int i = threadIdx.x; i < D / 2; i += blockDim.x)
      s_theta[i] = exp2(-(2.0 * (double)i / (double)D) * a.rope_log2_base);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int q = lane >> 2, l = lane & 3, n16 = lane & 15, g = lane >> 4;
  const uint32_t stage = mat + (uint32_t)((128 + 16 * wave) * kDensePitch);
  const int64_t th = a.tokens * a.heads, n_vec = a.rows * th, n_items = (n_vec + 15) / 16;
  const int LB = (QUANT == Q_MINMAX) ? a.group_log2 - 5 : 0;
  const int64_t ngroups = (QUANT == Q_MINMAX) ? (D >> a.group_log2) : 0;
  constexpr int NT = (1 << BITS) - 1;
  float tau[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) tau[i] = (QUANT == Q_LLOYD) ? 0.5f * (a.codebook[i] + a.codebook[i + 1]) : 0.0f;
  for (int64_t it = (int64_t)blockIdx.x * kDenseWaves + wave; it < n_items; it += (int64_t)gridDim.x * kDenseWaves) {
    const int64_t vec0 = it * 16, nvalid = min((int64_t)16, n_vec - vec0);
    const int64_t vec = min(vec0 + q, n_vec - 1);  // lanes past the end read the last vector; their stores drop
    const int64_t r = vec / th, rem = vec - r * th, t = rem / a.heads, h = rem - t * a.heads;
    RawRow<DT> raw;
    load_row<DT>(raw, reinterpret_cast<const char*>(a.x) + (r * a.sr + t * a.st + h * a.sh + 32 * l) * ES);
    float v[32];
    widen_row<DT>(raw, v);
    if (a.rope) {
      const int64_t pos = a.pos_offset + t;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        float c, sn;
        rope_cos_sin(pos, s_theta[16 * l + m], &c, &sn);
        const float x0 = v[2 * m], x1 = v[2 * m + 1];
        v[2 * m] = __builtin_fmaf(x0, c, -x1 * sn);
        v[2 * m + 1] = __builtin_fmaf(x0, sn, x1 * c);
      }
    }
    if constexpr (QUANT == Q_LLOYD) {
      const float rho = norm_separate<LV>(v);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(rho), make_buf_item(a.norm + vec0, (uint32_t)(4 * nvalid)),
                                            4u * (uint32_t)q, 0, 0);
    }
    dense_rotate_lane(v, mat, stage, q, l, n16, g);
    LaneCodes<BITS> cw;
    if constexpr (QUANT == Q_MINMAX) {
      uint32_t zb, sb;
      minmax_codes_lane<BITS, false>(v, 1.0f, LB, zb, sb, cw);
      const uint32_t go = 2u * (uint32_t)(q * ngroups + (l >> LB));
      const uint32_t gbytes = (uint32_t)(2 * nvalid * ngroups);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)sb, make_buf_item(a.scale + vec0 * ngroups, gbytes), go, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)zb, make_buf_item(a.zero + vec0 * ngroups, gbytes), go, 0, 0);
    } else {
      lloyd_codes_lane<BITS>(v, 1.0f, tau, cw);
    }
    store_lane_codes<BITS>(make_buf_item(a.codes + vec0 * CB, (uint32_t)(CB * nvalid)),
                           (uint32_t)(q * CB + l * (4 * BITS)), cw);
  }
}

template <int ODT, int BITS, int QUANT>
__global__ void __launch_bounds__(64 * kDenseWaves) decode_dense_kernel(const CodecArgs a) {
  constexpr int D = 128, CB = D * BITS / 8;
  constexpr int OES = (ODT == DT_F32) ? 4 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t s_dense[kDenseLds];
  __shared__ float s_cb[kMaxCodebook];
  const uint32_t mat = lds_addr(s_dense);
  dense_load_matrix<true>(a, mat);
  if constexpr (QUANT == Q_LLOYD) {
    if (threadIdx.x < (1 << BITS)) s_cb[threadIdx.x] = a.codebook[threadIdx.x];
  }
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int q = lane >> 2, l = lane & 3, n16 = lane & 15, g = lane >> 4;
  const uint32_t stage = mat + (uint32_t)((128 + 16 * wave) * kDensePitch);
  const int64_t n_vec = a.rows * a.tokens * a.heads, n_items = (n_vec + 15) / 16;
  const int LB = (QUANT == Q_MINMAX) ? a.group_log2 - 5 : 0;
  const int64_t ngroups = (QUANT == Q_MINMAX) ? (D >> a.group_log2) : 0;
  for (int64_t it = (int64_t)blockIdx.x * kDenseWaves + wave; it < n_items; it += (int64_t)gridDim.x * kDenseWaves) {
    const int64_t vec0 = it * 16, nvalid = min((int64_t)16, n_vec - vec0);
    LaneCodes<BITS> c;
    load_lane_codes<BITS>(make_buf(a.codes + vec0 * CB, CB * nvalid), (uint32_t)(q * CB + l * (4 * BITS)), c);
    float v[32];
    if constexpr (QUANT == Q_MINMAX) {
      const uint32_t go = 2u * (uint32_t)(q * ngroups + (l >> LB));
      const int64_t gbytes = 2 * nvalid * ngroups;
      const float sc = f16_value(__builtin_amdgcn_raw_buffer_load_b16(make_buf(a.scale + vec0 * ngroups, gbytes), go, 0, 0));
      const float z = f16_value(__builtin_amdgcn_raw_buffer_load_b16(make_buf(a.zero + vec0 * ngroups, gbytes), go, 0, 0));
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf((float)code_at<BITS>(c, i), sc, z);
    } else {
      // the norm scales the levels before the (linear) inverse rotation
      const float rho = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(make_buf(a.norm + vec0, 4 * nvalid), 4u * (uint32_t)q, 0, 0));
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = s_cb[code_at<BITS>(c, i)] * rho;
    }
    dense_rotate_lane(v, mat, stage, q, l, n16, g);
    // the lane's 32 outputs of vector vec0 + q, channels 32 l ..: 64 or 128 contiguous bytes
    const buf_t ob = make_buf_item(reinterpret_cast<char*>(a.y) + vec0 * D * OES, (uint32_t)(nvalid * D * OES));
    const uint32_t off = (uint32_t)((q * D + 32 * l) * OES);
    if constexpr (ODT == DT_F32) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]),
                                                       __float_as_uint(v[4 * k + 2]), __float_as_uint(v[4 * k + 3])},
                                               ob, off + 16u * k, 0, 0);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        u32x4_t w;
        if constexpr (ODT == DT_BF16) {
          w = u32x4_t{pack_bf16x2(v[8 * k], v[8 * k + 1]), pack_bf16x2(v[8 * k + 2], v[8 * k + 3]),
                      pack_bf16x2(v[8 * k + 4], v[8 * k + 5]), pack_bf16x2(v[8 * k + 6], v[8 * k + 7])};
        } else {
          w = u32x4_t{pack_f16x2(v[8 * k], v[8 * k + 1]), pack_f16x2(v[8 * k + 2], v[8 * k + 3]),
                      pack_f16x2(v[8 * k + 4], v[8 * k + 5]), pack_f16x2(v[8 * k + 6], v[8 * k + 7])};
        }
        __builtin_amdgcn_raw_buffer_store_b128(w, ob, off + 16u * k, 0, 0);
      }
    }
  }
}

// Grid of a sink pass: one sub-wavefront per sink vector of the call.
inline unsigned sink_blocks(const CodecArgs& a, int lv) {
  const int64_t n = (int64_t)a.n_sink - a.pos_offset;
  const int64_t nt = n <= 0 ? 0 : (n < a.tokens ? n : a.tokens);
  const int64_t nvec = a.rows * nt * a.heads;
  const int64_t per_block = 64 * kWavesPerBlock / lv;
  return (unsigned)((nvec + per_block - 1) / per_block);
}

// ---------------------------------------------------------------------------
// DECODE-STEP ATTENTION OVER THE ENCODED CACHE (d = 128, Walsh-Hadamard + min-max)
// ---------------------------------------------------------------------------
// A decoded key is P^T M y with the orthonormal Hadamard M = H / sqrt(128), the keys'
// permutation P and y = zero + code * scale per group, so q . k = (M P q) . y: each query
// is rotated once and scored against the stored codes, scale and zero directly.  Values
// are summed in the rotated domain, sum_t p_t P^T M y_t = P^T M sum_t p_t y_t, and rotated
// back once per output.  Sink slots hold fp16 of the unrotated vectors and are scored and
// summed unrotated.  Three passes: rotate the queries; per (row, KV head, chunk of slots)
// a partial softmax-weighted sum; per (row, query head) the merge of the chunks, the
// rotation back, the sinks and the normalisation.
constexpr float kInvSqrt128 = 0.08838834764831845f;

// Unnormalised Walsh-Hadamard transform (Sylvester order) of 128 values held by a wave as
// v0 = x[lane], v1 = x[lane + 64]: index bit 6 in the lane, bits 0..5 across lanes (7 stages
// of the butterfly network, 14 additions per lane).
__device__ __forceinline__ void fwht128_wave(float& v0, float& v1, int lane) {
  const float a = v0, b = v1;
  v0 = a + b;
  v1 = a - b;
#pragma unroll
  for (int bit = 1; bit < 64; bit <<= 1) {
    const float p0 = __shfl_xor(v0, bit), p1 = __shfl_xor(v1, bit);
    v0 = (lane & bit) ? p0 - v0 : v0 + p0;
    v1 = (lane & bit) ? p1 - v1 : v1 + p1;
  }
}

// rotated queries M P q: one wave per (row, query head); lane i holds channels i and i + 64
__global__ void __launch_bounds__(256) attend_rotate_q(const AttendArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= a.rows * a.q_heads) return;  // wave-uniform; no block barrier in this kernel
  const float* q = a.q + w * 128;
  // (P q)[k] = q[perm[k]]
  float z0 = q[a.use_perm_k ? a.perm_k[lane] : lane], z1 = q[a.use_perm_k ? a.perm_k[lane + 64] : lane + 64];
  fwht128_wave(z0, z1, lane);
  a.qrot[w * 128 + lane] = z0 * kInvSqrt128;
  a.qrot[w * 128 + lane + 64] = z1 * kInvSqrt128;
}

template <int BITS>
struct AttSlot {
  uint32_t kw[BITS / 2], vw[BITS / 2];  // the lane's 16 codes of the key and of the value
  uint32_t ks, kz, vs, vz;              // fp16 bits of the lane's group scale and zero
};

// Partial attention: one wave per (row, KV head, chunk of slots).  Lane (tk, l) =
// (lane / 8, lane % 8) holds channels 16 l .. 16 l + 15 of the token slot tk of each step of
// 8 slots; the 8 lanes of a slot reduce its scores, and each slot keeps its own running
// maximum, denominator and rotated-domain sums until the wave merges them at the end.
template <int BITS, int QG>
__global__ void __launch_bounds__(256) attend_partial(const AttendArgs a) {
  // the rotated query slices live in LDS (read every step) instead of 16 * QG registers
  __shared__ __attribute__((aligned(16))) float s_qv[4][QG * 128];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= a.rows * a.heads * a.n_chunks) return;  // wave-uniform; no block barrier follows
  const int64_t c = w % a.n_chunks, rh = w / a.n_chunks, h = rh % a.heads, r = rh / a.heads;
  const int tk = lane >> 3, l = lane & 7;
  int64_t len = a.tokens;
  if (a.lengths) {
    const int64_t n = a.lengths[r];
    len = n < 0 ? 0 : (n > a.tokens ? a.tokens : n);
  }
  const int64_t t_begin = max(c * (int64_t)a.chunk, (int64_t)a.n_sink);
  const int64_t t_end = min((c + 1) * (int64_t)a.chunk, len);
  const int64_t ngroups = 128 >> a.group_log2;
  const int g = (16 * l) >> a.group_log2;  // the lane's 16 channels lie in one group (G >= 32)
  constexpr int CB = 128 * BITS / 8;       // code bytes per vector
  constexpr int LB = 2 * BITS;             // code bytes per lane (16 codes)

  float sl[QG];
  {
    const float* src = a.qrot + (r * a.q_heads + h * QG) * 128;
    for (int i = lane; i < QG * 128; i += 64) s_qv[wave][i] = src[i];
    wave_lds_sync();
  }
  const uint32_t qaddr = lds_addr(&s_qv[wave][16 * l]);
#pragma unroll
  for (int m = 0; m < QG; ++m) {
    sl[m] = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4_t v = lds_ld4(qaddr + 512u * m + 16u * k);
      sl[m] += (__uint_as_float(v.x) + __uint_as_float(v.y)) + (__uint_as_float(v.z) + __uint_as_float(v.w));
    }
  }
  float mx[QG], ls[QG], zs[QG], acc[QG][16];
#pragma unroll
  for (int m = 0; m < QG; ++m) {
    mx[m] = -INFINITY;
    ls[m] = 0.0f;
    zs[m] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[m][i] = 0.0f;
  }

  // the lane's slot of step t0 (clamped into the chunk for the loads; masked afterwards)
  auto load = [&](int64_t t0, AttSlot<BITS>& s) __attribute__((always_inline)) {
    int64_t t = t0 + tk;
    if (t >= t_end) t = t_end - 1;
    const int64_t vec = (r * a.tokens + t) * a.heads + h;
    const uint32_t* kp = reinterpret_cast<const uint32_t*>(a.k_codes + vec * CB + l * LB);
    const uint32_t* vp = reinterpret_cast<const uint32_t*>(a.v_codes + vec * CB + l * LB);
#pragma unroll
    for (int i = 0; i < BITS / 2; ++i) {
      s.kw[i] = kp[i];
      s.vw[i] = vp[i];
    }
    s.ks = a.k_scale[vec * ngroups + g];
    s.kz = a.k_zero[vec * ngroups + g];
    s.vs = a.v_scale[vec * ngroups + g];
    s.vz = a.v_zero[vec * ngroups + g];
  };
  // codes to floats: spread each word's codes over bytes, then one byte-to-float conversion
  // per code (v_cvt_f32_ubyteN)
  auto unpack = [&](const uint32_t* wd, float* code) __attribute__((always_inline)) {
    constexpr int PER = 32 / BITS;         // codes per word
    constexpr int SPR = 8 / BITS;          // byte-spread words per word
    constexpr uint32_t BM = (BITS == 2) ? 0x03030303u : 0x0F0F0F0Fu;
#pragma unroll
    for (int j = 0; j < BITS / 2; ++j)
#pragma unroll
      for (int k = 0; k < SPR; ++k) {
        uint32_t e = (wd[j] >> (BITS * k)) & BM;  // byte b holds code SPR * b + k of word j
        asm volatile("" : "+v"(e));                // (kept whole, so each byte converts directly)
#pragma unroll
        for (int b = 0; b < 4; ++b) code[PER * j + SPR * b + k] = (float)((e >> (8 * b)) & 0xffu);
      }
  };

  if (t_begin < t_end) {
    AttSlot<BITS> cur, nxt;
    load(t_begin, cur);
    for (int64_t t0 = t_begin; t0 < t_end; t0 += 8) {
      if (t0 + 8 < t_end) load(t0 + 8, nxt);  // wave-uniform: the next step's loads in flight
      const bool valid = t0 + tk < t_end;
      float code[16];
      unpack(cur.kw, code);
      const float ks = f16_value(cur.ks), kz = f16_value(cur.kz);
      float s[QG];
      uint32_t qa = qaddr;
      asm volatile("" : "+v"(qa));  // read the slices here, each step (not hoisted into registers)
#pragma unroll
      for (int m = 0; m < QG; ++m) {
        float d = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const u32x4_t v = lds_ld4(qa + 512u * m + 16u * k);
          d = __builtin_fmaf(__uint_as_float(v.x), code[4 * k + 0], d);
          d = __builtin_fmaf(__uint_as_float(v.y), code[4 * k + 1], d);
          d = __builtin_fmaf(__uint_as_float(v.z), code[4 * k + 2], d);
          d = __builtin_fmaf(__uint_as_float(v.w), code[4 * k + 3], d);
        }
        float part = __builtin_fmaf(ks, d, kz * sl[m]);  // q~ . (zero + code * scale) over 16 channels
        part = add_x1(part);
        part = add_x2(part);
        part = add_half_mirror(part);
        s[m] = valid ? part * a.scale : -INFINITY;
      }
      // online softmax: rescale the slot's sums when its maximum grows
      bool grow = false;
      float mn[QG];
#pragma unroll
      for (int m = 0; m < QG; ++m) {
        mn[m] = fmaxf(mx[m], s[m]);
        grow |= mn[m] > mx[m];
      }
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
        for (int m = 0; m < QG; ++m) {
          const float corr = (mn[m] > mx[m]) ? __expf(mx[m] - mn[m]) : 1.0f;
          ls[m] *= corr;
          zs[m] *= corr;
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[m][i] *= corr;
          mx[m] = mn[m];
        }
      }
      unpack(cur.vw, code);
      const float vs = f16_value(cur.vs), vz = f16_value(cur.vz);
#pragma unroll
      for (int m = 0; m < QG; ++m) {
        const float p = valid ? __expf(s[m] - mx[m]) : 0.0f;
        ls[m] += p;
        zs[m] = __builtin_fmaf(p, vz, zs[m]);  // sum_t p_t zero_t, applies to every channel of the group
        const float ps = p * vs;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][i] = __builtin_fmaf(ps, code[i], acc[m][i]);
      }
      cur = nxt;
    }
  }
  // merge the wave's 8 slots and write the chunk's partial
#pragma unroll
  for (int m = 0; m < QG; ++m) {
    float M = mx[m];
    M = fmaxf(M, __shfl_xor(M, 8));
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float f = (mx[m] == -INFINITY) ? 0.0f : __expf(mx[m] - M);
    float L = ls[m] * f;
    L += __shfl_xor(L, 8);
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    float* pb = a.part + ((r * a.q_heads + h * QG + m) * a.n_chunks + c) * kAttendPart;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = (acc[m][i] + zs[m]) * f;
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (tk == 0) pb[16 * l + i] = v;
    }
    if (lane == 0) {
      pb[128] = M;
      pb[129] = L;
    }
  }
}

// Partial attention on the int8 matrix cores, for 2-bit codes with one group of 128 channels
// (scale and zero per vector).  Every product is exact integer arithmetic:
//  * keys: a code byte is spread into the bytes of four words by masks, so byte e holds
//    code(e) * mul(e) with mul in {1, 4, 16, 16}; the rotated query of each head is scaled by
//    a power of two, divided by mul and rounded to a 31-bit integer, cut into four signed
//    8-bit digits (rows 4 m + s of the A operand), so one 16x16x64 product per 64 channels
//    gives per digit the integer dot product of 16 slots, recombined in fp32;
//  * values: per window of slots, the key pass scores every slot first (the scores stay in
//    registers) and updates the running maximum; then each lane turns its own slots' weights
//    p * scale_v, relative to that maximum and scaled by a power of two to at most 2^27, into
//    integers in LDS, which the value product reads as four signed 8-bit digits (columns 4 m + s
//    of the B operand); the value codes of 64 slots, staged in LDS and read back transposed
//    (16-bit halves regrouped by byte permutes), are the A operand.  The integer sums are
//    turned into floats when the running maximum or the weight scale changes, every 1024
//    windows (int32 headroom), and at the end of the chunk.
// Lanes: n16 = lane % 16 and g = lane / 16 as in the operand layouts; in the key product
// lane (n16, g) holds slot n16 of a 16-slot block for head g; in the value product lane
// (4 m + s, g) holds digit s of head m for channels 32 g + 8 j + b (register j, product b).
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));
constexpr int kMmaW = 128;  // slots per window (a multiple of 64)
constexpr int kMmaPad = 16;  // padding of the LDS weight-integer rows (banks of the row writes)
template <int K>
__device__ __forceinline__ uint32_t code_bytes(uint32_t x) {  // code 4 b + K of byte b, times code_mul(K)
  if constexpr (K < 3) return x & (0x03030303u << (2 * K));
  else return (x >> 2) & 0x30303030u;
}
__host__ __device__ constexpr int code_mul(int k) { return k == 0 ? 1 : (k == 1 ? 4 : 16); }

// Tasks are (row, chunk, head) with the head fastest; blocks take 4 consecutive tasks, and
// blocks 16 k + x and 16 k + 8 + x (x < 8) take consecutive task quads, so that both halves
// of the heads of a (row, chunk) are read on one XCD (blocks go round-robin over the 8 XCDs)
// and share its L2 for the scale planes.  Per window of 128 slots: the value codes go to LDS
// (16-byte loads), the key product scores the slots (lane (n16, g): slot n16 of each 16-slot
// block, head g), the window maximum decides a flush, each lane turns its scores into weight
// integers in LDS, and the value product reads them as digits.  Code and scale planes are
// read through descriptors sized to the window's valid slots: reads past them return zeros.
// Reductions over the 16 lanes of each row (every lane gets its row's result) with DPP:
// quad permutes for lanes xor 1 and xor 2, row rotations by 4 and 8.
__device__ __forceinline__ float dpp_f(float v, int ctrl) {
  switch (ctrl) {  // the control must be a constant of the builtin
    case 0xB1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    case 0x4E: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    case 0x124: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  }
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f(v, 0xB1));
  v = fmaxf(v, dpp_f(v, 0x4E));
  v = fmaxf(v, dpp_f(v, 0x124));
  return fmaxf(v, dpp_f(v, 0x128));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f(v, 0xB1);
  v += dpp_f(v, 0x4E);
  v += dpp_f(v, 0x124);
  return v + dpp_f(v, 0x128);
}
// the value of row m (lanes 16 m .. 16 m + 15 hold it), wave-uniform
__device__ __forceinline__ float row_value(float v, int m) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * m));
}

// A weight integer N < 2^27 as four balanced signed 8-bit digits, one per byte:
// N = sum_s d_s 256^s with d_0..d_2 in [-128, 127] (bytes of N + 0x808080, minus 128) and
// d_3 = (N + 0x808080) >> 24 in [0, 8].
__device__ __forceinline__ uint32_t weight_digits(uint32_t n) { return (n + 0x808080u) ^ 0x808080u; }

// The eight value products of a 64-slot group: A = the codes of channel 8 n16 + b spread by
// code_bytes (X: channels 8 n16 .. +3, Y: 8 n16 + 4 .. +7; byte j of word bt = slot j of
// block bt), B = the weight digits bop.
__device__ __forceinline__ void value_product(const uint32_t (&X)[4], const uint32_t (&Y)[4], const i32x4_t& bop,
                                              i32x4_t (&cv)[8]) {
#define KVQ_VPROD(B, SRC, K)                                                                        \
  {                                                                                                 \
    const i32x4_t ap = {(int32_t)code_bytes<K>(SRC[0]), (int32_t)code_bytes<K>(SRC[1]),             \
                        (int32_t)code_bytes<K>(SRC[2]), (int32_t)code_bytes<K>(SRC[3])};            \
    cv[B] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ap, bop, cv[B], 0, 0, 0);                         \
  }
  KVQ_VPROD(0, X, 0)
  KVQ_VPROD(1, X, 1)
  KVQ_VPROD(2, X, 2)
  KVQ_VPROD(3, X, 3)
  KVQ_VPROD(4, Y, 0)
  KVQ_VPROD(5, Y, 1)
  KVQ_VPROD(6, Y, 2)
  KVQ_VPROD(7, Y, 3)
#undef KVQ_VPROD
}

// Query side of the key product for (row r, KV head h): A operands qa (lane (4 m + s, g),
// product u, byte e: digit s of head m's scaled query, channel 16 (2 g + u) + 4 (e % 4) + e / 4),
// and for the lane's key-product head g the factors of score = k_scale raw rs + k_zero zq
// (log2 units).
template <int QG, int BITS = 2>
__device__ __forceinline__ void mma_query(const AttendArgs& a, const float* qb, int lane, i32x4_t (&qa)[2],
                                          float& rs, float& zq) {
  const int n16 = lane & 15, g = lane >> 4, qm = n16 >> 2, qs = n16 & 3;
  constexpr float kLog2e = 1.4426950408889634f;
  // per-head max |q~| and sum q~ of the rotated queries qb[m * 128 + c] (m < QG)
  float qmx[4], qsum[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float v0 = m < QG ? qb[m * 128 + lane] : 0.0f, v1 = m < QG ? qb[m * 128 + lane + 64] : 0.0f;
    const float x = row_max16(fmaxf(fabsf(v0), fabsf(v1))), y = row_sum16(v0 + v1);
    qmx[m] = fmaxf(fmaxf(row_value(x, 0), row_value(x, 1)), fmaxf(row_value(x, 2), row_value(x, 3)));
    qsum[m] = (row_value(y, 0) + row_value(y, 1)) + (row_value(y, 2) + row_value(y, 3));
  }
  // query scale 2^e with 16 |q~| 2^e < 2^30
  float qsc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    int ex;
    (void)__builtin_frexpf(16.0f * qmx[m], &ex);
    qsc[m] = __builtin_ldexpf(1.0f, 30 - ex);
  }
  // A operand of the key product: lane (4 m + s, g), product u, byte e holds digit s of the
  // scaled query of channel 16 (2 g + u) + 4 (e % 4) + e / 4
  {
    const float sqm = qm == 0 ? qsc[0] : (qm == 1 ? qsc[1] : (qm == 2 ? qsc[2] : qsc[3]));
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float qv[16];
      // the 16 channels of product u in lane group g: 2-bit, 16 (2 g + u) + 4 (e % 4) + e / 4;
      // 4-bit, 32 g + 16 u + 8 (e / 8) + 2 (e % 4) + (e / 4) % 2
      const float* src = qb + qm * 128 + 16 * (2 * g + u);
#pragma unroll
      for (int i = 0; i < 16; ++i) qv[i] = qm < QG ? src[i] : 0.0f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t word = 0;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int e = 4 * d + bb;
          const int ci = BITS == 2 ? 4 * (e & 3) + (e >> 2) : 8 * (e >> 3) + 2 * (e & 3) + ((e >> 2) & 1);
          const float mul = BITS == 2 ? (float)(16 / code_mul(e >> 2)) : 16.0f;
          const int32_t Q = (int32_t)__builtin_rintf(qv[ci] * mul * sqm);
          // balanced base-256 digits: T = Q + 0x808080, digit s = byte s of T - 128 (s < 3), T >> 24 (s = 3)
          const int32_t T = Q + 0x808080;
          const uint32_t byte = ((uint32_t)(T >> (8 * qs)) & 0xffu) ^ (qs < 3 ? 0x80u : 0u);
          word |= byte << (8 * bb);
        }
        qa[u][d] = (int32_t)word;
      }
    }
  }
  // key-product lane role: head g; score = (k_scale * raw * rs + k_zero * zq) in log2 units
  const float sc2 = a.scale * kLog2e;
  const float sqg = g == 0 ? qsc[0] : (g == 1 ? qsc[1] : (g == 2 ? qsc[2] : qsc[3]));
  rs = sc2 / (16.0f * sqg);
  zq = g < QG ? sc2 * (g == 0 ? qsum[0] : (g == 1 ? qsum[1] : (g == 2 ? qsum[2] : qsum[3]))) : 0.0f;
}

template <int QG>
__global__ void __launch_bounds__(256) attend_partial_mma(const AttendArgs a) {
  __shared__ __attribute__((aligned(16))) float4 s_sc[4][kMmaW];                // k scale, k zero, v scale, v zero
  __shared__ __attribute__((aligned(16))) uint32_t s_n[4][4][kMmaW + kMmaPad];  // weight integers per head
  __shared__ __attribute__((aligned(16))) uint8_t s_vc[4][kMmaW * 40];          // value codes, slot s at 32 s + 32 (s / 4)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t blk = blockIdx.x;
  const int64_t quad = (blk >> 4) * 16 + ((blk & 7) << 1) + ((blk >> 3) & 1);
  const int64_t w = quad * 4 + wave;
  if (w >= a.rows * a.heads * a.n_chunks) return;  // wave-uniform; no block barrier in this kernel
  const int64_t h = w % a.heads, rc = w / a.heads, c = rc % a.n_chunks, r = rc / a.n_chunks;
  int64_t len = a.tokens;
  if (a.lengths) {
    const int64_t n = a.lengths[r];
    len = n < 0 ? 0 : (n > a.tokens ? a.tokens : n);
  }
  const int64_t t_begin = max(c * (int64_t)a.chunk, (int64_t)a.n_sink);
  const int64_t t_end = min((c + 1) * (int64_t)a.chunk, len);
  const int n16 = lane & 15, g = lane >> 4;
  const int qm = n16 >> 2, qs = n16 & 3;  // head and digit of the lane's column in the value product
  float4* const sc = &s_sc[wave][0];
  uint32_t* const sn = &s_n[wave][0][0];
  uint8_t* const vc = &s_vc[wave][0];
  constexpr int SR = kMmaW + kMmaPad;
  
  i32x4_t qa[2];
  float rs, zq;
  mma_query<QG>(a, a.qrot + (r * a.q_heads + h * QG) * 128, lane, qa, rs, zq);

  i32x4_t cv[8];
  float fo[8];  // value product: channels 32 g + 8 qs + b of head qm, summed over the digits
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    fo[b] = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) cv[b][j] = 0;
  }
  float Mrun = -INFINITY;      // running maximum of head g (log2 units)
  float Lp = 0.0f, Zp = 0.0f;  // head g, the lane's slots: pending sums of p 2^E and p 2^E v_zero
  float Lf = 0.0f, Zf = 0.0f;
  int Ecur = 0, since = 0;
  bool first = true;
  // integer sums to floats: weight each digit, sum the 4 digit lanes, keep register j = qs
  auto flush = [&](float corr) __attribute__((always_inline)) {
    const float corr_m = __shfl(corr, 16 * qm);  // the factor of head qm
    const float kb = __builtin_ldexpf(1.0f, 8 * qs - Ecur);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const float k = kb * (1.0f / (float)code_mul(b & 3));
      float add = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v = (float)cv[b][j] * k;
        v = add_x1(v);
        v = add_x2(v);
        add = qs == j ? v : add;
        cv[b][j] = 0;
      }
      fo[b] = (fo[b] + add) * corr_m;
    }
    const float le = __builtin_ldexpf(1.0f, -Ecur);
    Lf = (Lf + Lp * le) * corr;
    Zf = (Zf + Zp * le) * corr;
    Lp = 0.0f;
    Zp = 0.0f;
  };

  const uint32_t sT = (uint32_t)a.heads * 32u;  // bytes between slots in a code plane
  const uint32_t sH2 = (uint32_t)a.heads * 2u;  // bytes between slots in a scale plane
  const int64_t rh0 = r * a.tokens * a.heads + h;
  const uint32_t koff = (uint32_t)n16 * sT + 8u * (uint32_t)g;   // key-code bytes of the lane in a block
  const uint32_t vrd = 160u * (uint32_t)g + 2u * (uint32_t)n16;  // LDS value codes: slot 4 g, bytes 2 n16
  const uint32_t dsel = (uint32_t)qs | ((uint32_t)qs + 4u) << 8;  // byte qs of two words -> bytes 0, 1
  // Loads of a window (value codes, scales, key codes) are issued one window ahead: the value
  // codes and scales of window w + 1 after window w's are staged in LDS, its key codes after
  // window w's key product.  Descriptors cover the valid slots of the window they serve; a
  // window at or past the end of the chunk gets empty descriptors (its loads read zeros).
  auto win_bytes = [&](int64_t w0, uint32_t per_slot, uint32_t tail) -> uint32_t {
    const int64_t n = min((int64_t)kMmaW, t_end - w0);
    return n > 0 ? (uint32_t)(n - 1) * per_slot + tail : 0u;
  };
  u32x4_t vq[kMmaW / 32];
  u32x2_t kq[kMmaW / 16];
  uint32_t sq[kMmaW / 64][4];
  auto load_vs = [&](int64_t w0) __attribute__((always_inline)) {  // value codes and scales
    const int64_t vw = rh0 + w0 * a.heads;
    const uint32_t cb = win_bytes(w0, sT, 32u), sb = win_bytes(w0, sH2, 2u);
    const buf_t bvc = make_buf(a.v_codes + vw * 32, cb);
    const buf_t bks = make_buf(a.k_scale + vw, sb), bkz = make_buf(a.k_zero + vw, sb);
    const buf_t bvs = make_buf(a.v_scale + vw, sb), bvz = make_buf(a.v_zero + vw, sb);
#pragma unroll
    for (int k = 0; k < kMmaW / 32; ++k) {
      const uint32_t cc = (uint32_t)(lane + 64 * k);
      vq[k] = __builtin_amdgcn_raw_buffer_load_b128(bvc, (cc >> 1) * sT + 16u * (cc & 1u), 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kMmaW / 64; ++k) {
      const uint32_t o = (uint32_t)(lane + 64 * k) * sH2;
      sq[k][0] = __builtin_amdgcn_raw_buffer_load_b16(bks, o, 0, 0);
      sq[k][1] = __builtin_amdgcn_raw_buffer_load_b16(bkz, o, 0, 0);
      sq[k][2] = __builtin_amdgcn_raw_buffer_load_b16(bvs, o, 0, 0);
      sq[k][3] = __builtin_amdgcn_raw_buffer_load_b16(bvz, o, 0, 0);
    }
  };
  auto load_k = [&](int64_t w0) __attribute__((always_inline)) {  // key codes, lane (n16, g)
    const int64_t vw = rh0 + w0 * a.heads;
    const buf_t bkc = make_buf(a.k_codes + vw * 32, win_bytes(w0, sT, 32u));
#pragma unroll
    for (int bk = 0; bk < kMmaW / 16; ++bk)
      kq[bk] = __builtin_amdgcn_raw_buffer_load_b64(bkc, koff + (uint32_t)(16 * bk) * sT, 0, 0);
  };
  if (t_begin < t_end) {
    load_vs(t_begin);
    load_k(t_begin);
  }
  for (int64_t wt0 = t_begin; wt0 < t_end; wt0 += kMmaW) {
    const int nv = (int)min((int64_t)kMmaW, t_end - wt0);  // valid slots of the window (>= 1); the
    // rest of a window reads zeros through the descriptors and is masked by its slot index
    float vsm = 0.0f;
#pragma unroll
    for (int k = 0; k < kMmaW / 64; ++k) {
      const int i = lane + 64 * k;
      const float vs = f16_value(sq[k][2]);
      sc[i] = make_float4(f16_value(sq[k][0]), f16_value(sq[k][1]), vs, f16_value(sq[k][3]));
      vsm = fmaxf(vsm, fabsf(vs));
    }
#pragma unroll
    for (int k = 0; k < kMmaW / 32; ++k) {
      const uint32_t cc = (uint32_t)(lane + 64 * k), sl = cc >> 1;
      *reinterpret_cast<u32x4_t*>(vc + 32u * sl + 32u * (sl >> 2) + 16u * (cc & 1u)) = vq[k];
    }
    load_vs(wt0 + kMmaW);
    wave_lds_sync();
    // pass 1: scores of the lane's slots (head g), window maximum per head; the products of
    // 4 blocks are issued before any is read
    float scv[kMmaW / 16];
    float mw = -INFINITY;
#pragma unroll
    for (int q4 = 0; q4 < kMmaW / 16; q4 += 4) {
      i32x4_t acc[4];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const u32x2_t kv = kq[q4 + bt];
        const i32x4_t b0 = {(int32_t)code_bytes<0>(kv.x), (int32_t)code_bytes<1>(kv.x), (int32_t)code_bytes<2>(kv.x),
                            (int32_t)code_bytes<3>(kv.x)};
        acc[bt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[0], b0, i32x4_t{0, 0, 0, 0}, 0, 0, 0);
      }
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const u32x2_t kv = kq[q4 + bt];
        const i32x4_t b1 = {(int32_t)code_bytes<0>(kv.y), (int32_t)code_bytes<1>(kv.y), (int32_t)code_bytes<2>(kv.y),
                            (int32_t)code_bytes<3>(kv.y)};
        acc[bt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[1], b1, acc[bt], 0, 0, 0);
      }
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const int i = 16 * (q4 + bt) + n16;
        // lane (n16, g) holds digits 0..3 of head g for slot i
        const float raw = __builtin_fmaf((float)acc[bt][3], 16777216.0f,
                                         __builtin_fmaf((float)acc[bt][2], 65536.0f,
                                                        __builtin_fmaf((float)acc[bt][1], 256.0f, (float)acc[bt][0])));
        const float4 s4 = sc[i];
        const float sco = __builtin_fmaf(s4.x * raw, rs, s4.y * zq);
        scv[q4 + bt] = i < nv ? sco : -INFINITY;
        mw = fmaxf(mw, scv[q4 + bt]);
      }
    }
    load_k(wt0 + kMmaW);
    mw = row_max16(mw);  // every lane of row g: the window maximum of head g
    vsm = row_max16(vsm);
    vsm = fmaxf(fmaxf(row_value(vsm, 0), row_value(vsm, 1)), fmaxf(row_value(vsm, 2), row_value(vsm, 3)));
    int ex;
    (void)__builtin_frexpf(vsm, &ex);
    const int Ew = 27 - ex;  // v_scale 2^Ew < 2^27 for every slot of the window
    const float Mnew = fmaxf(Mrun, mw);
    const bool grow = __builtin_amdgcn_ballot_w64(Mnew > Mrun) != 0;
    if (grow || first || Ew < Ecur || since >= 1024) {  // wave-uniform
      flush(__builtin_amdgcn_exp2f(Mrun - Mnew));
      Mrun = Mnew;
      Ecur = Ew;
      since = 0;
      first = false;
    }
    ++since;
    // pass 1.5: weight integers p v_scale 2^E of the lane's slots, sums of p and p v_zero
    const float Mk = Mrun - (float)Ecur;  // p 2^E = exp2(s - Mk)
#pragma unroll
    for (int bk = 0; bk < kMmaW / 16; ++bk) {
        const int i = 16 * bk + n16;
        const float pe = __builtin_amdgcn_exp2f(scv[bk] - Mk);
        const float4 s4 = sc[i];
        Lp += pe;
        Zp = __builtin_fmaf(pe, s4.w, Zp);
        sn[g * SR + i] = weight_digits((uint32_t)__builtin_fmaf(pe, s4.z, 0.5f));
      }
    wave_lds_sync();
    // pass 2: value product per 64-slot group
#pragma unroll
    for (int q4 = 0; q4 < kMmaW / 16; q4 += 4) {
      {
        uint32_t D[4], X[4], Y[4];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          const int i0 = 16 * (q4 + bt) + 4 * g;  // window slot of the lane's 4 slots
          const u32x4_t nw = *reinterpret_cast<const u32x4_t*>(&sn[qm * SR + i0]);
          D[bt] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(nw.w, nw.z, dsel), __builtin_amdgcn_perm(nw.y, nw.x, dsel),
                                        0x05040100u);  // byte j: digit qs of slot i0 + j
          const uint8_t* p0 = vc + vrd + 640u * (uint32_t)(q4 + bt);
          u16x2_t lo, hi;
          lo[0] = *reinterpret_cast<const uint16_t*>(p0);
          lo[1] = *reinterpret_cast<const uint16_t*>(p0 + 32);
          hi[0] = *reinterpret_cast<const uint16_t*>(p0 + 64);
          hi[1] = *reinterpret_cast<const uint16_t*>(p0 + 96);
          const uint32_t lw = __builtin_bit_cast(uint32_t, lo), hw = __builtin_bit_cast(uint32_t, hi);
          X[bt] = __builtin_amdgcn_perm(hw, lw, 0x06040200u);  // byte j: channels 8 n16 .. +3 of slot j
          Y[bt] = __builtin_amdgcn_perm(hw, lw, 0x07050301u);  // byte j: channels 8 n16 + 4 .. +7
        }
        const i32x4_t bop = {(int32_t)D[0], (int32_t)D[1], (int32_t)D[2], (int32_t)D[3]};
        value_product(X, Y, bop, cv);
      }
    }
    wave_lds_sync();
  }
  if (t_begin < t_end) flush(1.0f);
  // sums of head g over the 16 slot lanes of row g, then head qm's for the output lanes
  Lf = row_sum16(Lf);
  Zf = row_sum16(Zf);
  const float Lm = __shfl(Lf, 16 * qm), Zm = __shfl(Zf, 16 * qm), Mm = __shfl(Mrun, 16 * qm);
  if (qm < QG) {
    float* pb = a.part + ((r * a.q_heads + h * QG + qm) * a.n_chunks + c) * kAttendPart;
#pragma unroll
    for (int b = 0; b < 8; ++b) pb[32 * g + 8 * qs + b] = fo[b] + Zm;  // channel 32 g + 8 qs + b
    if (qs == 0 && g == 0) {
      pb[128] = (t_begin < t_end) ? Mm * 0.6931471805599453f : -INFINITY;
      pb[129] = Lm;
    }
  }
}

// The same pass with the 4 waves of a block on 4 consecutive KV heads of one (row, chunk), for
// caches whose head count is a multiple of 4: the block loads each 64-slot window's code rows of
// its 4 heads (128 contiguous bytes per slot and plane, whole 128-byte lines) and their scales
// into LDS once, and each wave computes its head from there.  The loads run one window ahead in
// registers (at the Llama-3 cache, with the chunks below, 3 % faster than two windows ahead and
// 2 % faster than one window of 128 slots: fewer bytes in flight stream faster here).  Rows of a code
// window are padded to 136 bytes: the key reads (8 bytes, slot n16 of a block) and the value
// reads (32-bit words, slots 4 g + j) then fall into distinct banks.  Chunk c of a row takes
// every n_chunks-th window from window c on (after the sink slots), so the blocks of a row
// stream neighbouring windows at the same time (measured 1.7 % faster at the Llama-3 cache
// than contiguous chunks of slots); the combine pass merges any split of the slots alike.
// Per code width: code bytes per head and slot, slots per window, LDS bytes per slot row.
template <int BITS> struct BlkGeo {
  static constexpr int CB = 16 * BITS;
  static constexpr int W = 64;
  static constexpr int ROWB = BITS == 2 ? 136 : 272;
};
// (at most 168 VGPRs, 3 waves per SIMD: measured 9 % faster than 2 at 232 VGPRs; 4 waves at 128
// VGPRs, with spills, measured 1 % slower)
template <int BITS, int QG>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) attend_partial_mma_blk(const AttendArgs a) {
  constexpr int CB = BlkGeo<BITS>::CB, WN = BlkGeo<BITS>::W, kRowB = BlkGeo<BITS>::ROWB;
  __shared__ __attribute__((aligned(16))) uint8_t s_kc[WN * kRowB];
  __shared__ __attribute__((aligned(16))) uint8_t s_vc[WN * kRowB];
  __shared__ __attribute__((aligned(16))) uint16_t s_sr[4][WN][4];          // (k scale, k zero, v scale, v zero), slot, head
  __shared__ __attribute__((aligned(16))) uint32_t s_n[4][4][WN + kMmaPad];  // per wave: weight integers per head
  __shared__ __attribute__((aligned(16))) float s_qr[4][QG * 128];             // per wave: its rotated queries
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t blk = blockIdx.x;
  const int64_t quad = (blk >> 4) * 16 + ((blk & 7) << 1) + ((blk >> 3) & 1);
  if (quad * 4 >= a.rows * a.heads * a.n_chunks) return;  // block-uniform: the task count is a multiple of 4
  const int64_t w = quad * 4 + wave;
  const int64_t h = w % a.heads, rc = w / a.heads, c = rc % a.n_chunks, r = rc / a.n_chunks;
  const int64_t h0 = h - wave;  // the block's first head (heads are a multiple of 4)
  int64_t len = a.tokens;
  if (a.lengths) {
    const int64_t n = a.lengths[r];
    len = n < 0 ? 0 : (n > a.tokens ? a.tokens : n);
  }
  const int64_t SW = a.n_chunks * (int64_t)WN;  // a chunk's windows: every n_chunks-th window of the row
  const int64_t t_begin = (int64_t)a.n_sink + c * (int64_t)WN;
  const int64_t t_end = len;
  const int n16 = lane & 15, g = lane >> 4;
  const int qm = n16 >> 2, qs = n16 & 3;
  uint32_t* const sn = &s_n[wave][0][0];
  constexpr int SR = WN + kMmaPad;

  // the wave's rotated queries M P q, computed here rather than by a pass of their own (the
  // same arithmetic as attend_rotate_q), into the wave's LDS slice
  {
    float* qr = s_qr[wave];
#pragma unroll
    for (int m = 0; m < QG; ++m) {
      const float* q = a.q + (r * a.q_heads + h * QG + m) * 128;
      float z0 = q[a.use_perm_k ? a.perm_k[lane] : lane], z1 = q[a.use_perm_k ? a.perm_k[lane + 64] : lane + 64];
      fwht128_wave(z0, z1, lane);
      qr[m * 128 + lane] = z0 * kInvSqrt128;
      qr[m * 128 + lane + 64] = z1 * kInvSqrt128;
    }
    wave_lds_sync();
  }
  i32x4_t qa[2];
  float rs, zq;
  mma_query<QG, BITS>(a, s_qr[wave], lane, qa, rs, zq);

  i32x4_t cv[8];
  float fo[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    fo[b] = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) cv[b][j] = 0;
  }
  float Mrun = -INFINITY, Lp = 0.0f, Zp = 0.0f, Lf = 0.0f, Zf = 0.0f;
  int Ecur = 0, since = 0;
  bool first = true;
  auto flush = [&](float corr) __attribute__((always_inline)) {
    const float corr_m = __shfl(corr, 16 * qm);
    const float kb = __builtin_ldexpf(1.0f, 8 * qs - Ecur);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const float k = BITS == 2 ? kb * (1.0f / (float)code_mul(b & 3)) : kb;
      float add = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v = (float)cv[b][j] * k;
        v = add_x1(v);
        v = add_x2(v);
        add = qs == j ? v : add;
        cv[b][j] = 0;
      }
      fo[b] = (fo[b] + add) * corr_m;
    }
    const float le = __builtin_ldexpf(1.0f, -Ecur);
    Lf = (Lf + Lp * le) * corr;
    Zf = (Zf + Zp * le) * corr;
    Lp = 0.0f;
    Zp = 0.0f;
  };

  const uint32_t sT = (uint32_t)a.heads * (uint32_t)CB, sH2 = (uint32_t)a.heads * 2u;
  const int64_t rb0 = r * a.tokens * a.heads + h0;  // vector index of (row, slot 0, head h0)
  constexpr int UPS = CB / 4;                       // 16-byte units per slot (4 heads)
  constexpr int NU = WN * UPS / 256;                // 16-byte units per thread and plane
  constexpr int NS = WN / 64;                       // scale slots per thread
  const int sp = tid >> 6;                          // the thread's scale plane
  const uint16_t* const splane = sp == 0 ? a.k_scale : (sp == 1 ? a.k_zero : (sp == 2 ? a.v_scale : a.v_zero));
  struct WinRegs {
    u32x4_t kq[NU], vq[NU];
    u32x2_t sq[NS];
  };
  WinRegs RA;
  auto load_win = [&](int64_t w0, WinRegs& R) __attribute__((always_inline)) {
    const int64_t vb = rb0 + w0 * a.heads;
    const int64_t n = min((int64_t)WN, t_end - w0);
    const uint32_t cb = n > 0 ? (uint32_t)(n - 1) * sT + 4u * CB : 0u, sb = n > 0 ? (uint32_t)(n - 1) * sH2 + 8u : 0u;
    const buf_t bkc = make_buf(a.k_codes + vb * CB, cb), bvc = make_buf(a.v_codes + vb * CB, cb);
    const buf_t bs = make_buf(splane + vb, sb);
    // the scales first: the key pass needs them first (measured 1 % faster than after the codes)
#pragma unroll
    for (int e = 0; e < NS; ++e) R.sq[e] = __builtin_amdgcn_raw_buffer_load_b64(bs, (uint32_t)(NS * (tid & 63) + e) * sH2, 0, 0);
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const uint32_t u = (uint32_t)(tid + 256 * k);  // slot u / UPS, bytes 16 (u % UPS) of the 4 heads' row
      const uint32_t off = (u / UPS) * sT + 16u * (u % UPS);
      // each code line is read once, by this block: streamed (non-temporal, system scope), which
      // measured 6-7 % faster than temporal loads at the Llama-3 cache; the scale records, half
      // of whose lines the block of the other head quad reads, stay temporal
      R.kq[k] = __builtin_amdgcn_raw_buffer_load_b128(bkc, off, 0, kNT | kSC1);
      R.vq[k] = __builtin_amdgcn_raw_buffer_load_b128(bvc, off, 0, kNT | kSC1);
    }
  };
  const uint32_t vsel = (n16 & 1) ? 0x07060302u : 0x05040100u;  // the lane's 16-bit half of two words
  const uint32_t dsel = (uint32_t)qs | ((uint32_t)qs + 4u) << 8;  // byte qs of two words -> bytes 0, 1
  if (t_begin < t_end) load_win(t_begin, RA);
  auto window = [&](int64_t wt0, WinRegs& R) __attribute__((always_inline)) {
    const int nv = (int)min((int64_t)WN, t_end - wt0);
    __syncthreads();  // every wave is done with the previous window's LDS
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const uint32_t u = (uint32_t)(tid + 256 * k), o = (u / UPS) * kRowB + 16u * (u % UPS);
      *reinterpret_cast<u32x2_t*>(s_kc + o) = u32x2_t{R.kq[k].x, R.kq[k].y};
      *reinterpret_cast<u32x2_t*>(s_kc + o + 8) = u32x2_t{R.kq[k].z, R.kq[k].w};
      *reinterpret_cast<u32x2_t*>(s_vc + o) = u32x2_t{R.vq[k].x, R.vq[k].y};
      *reinterpret_cast<u32x2_t*>(s_vc + o + 8) = u32x2_t{R.vq[k].z, R.vq[k].w};
    }
#pragma unroll
    for (int e = 0; e < NS; ++e) *reinterpret_cast<u32x2_t*>(&s_sr[sp][NS * (tid & 63) + e][0]) = R.sq[e];
    __syncthreads();
    load_win(wt0 + SW, R);  // the chunk's next window
    float vsm = 0.0f;
#pragma unroll
    for (int k = 0; k < NS; ++k) vsm = fmaxf(vsm, fabsf(f16_value(s_sr[2][lane + 64 * k][wave])));
    // pass 1: key product from LDS
    float scv[WN / 16];
    float mw = -INFINITY;
#pragma unroll
    for (int q4 = 0; q4 < WN / 16; q4 += 4) {
      i32x4_t acc[4];
      if constexpr (BITS == 2) {
        u32x2_t kv[4];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          kv[bt] = *reinterpret_cast<const u32x2_t*>(s_kc + (16 * (q4 + bt) + n16) * kRowB + CB * wave + 8 * g);
          const i32x4_t b0 = {(int32_t)code_bytes<0>(kv[bt].x), (int32_t)code_bytes<1>(kv[bt].x),
                              (int32_t)code_bytes<2>(kv[bt].x), (int32_t)code_bytes<3>(kv[bt].x)};
          acc[bt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[0], b0, i32x4_t{0, 0, 0, 0}, 0, 0, 0);
        }
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          const i32x4_t b1 = {(int32_t)code_bytes<0>(kv[bt].y), (int32_t)code_bytes<1>(kv[bt].y),
                              (int32_t)code_bytes<2>(kv[bt].y), (int32_t)code_bytes<3>(kv[bt].y)};
          acc[bt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[1], b1, acc[bt], 0, 0, 0);
        }
      } else {  // 4-bit: a word's codes 2 b (low nibbles) and 2 b + 1 (high nibbles)
        u32x4_t kv[4];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          kv[bt] = *reinterpret_cast<const u32x4_t*>(s_kc + (16 * (q4 + bt) + n16) * kRowB + CB * wave + 16 * g);
          const i32x4_t b0 = {(int32_t)(kv[bt].x & 0x0F0F0F0Fu), (int32_t)((kv[bt].x >> 4) & 0x0F0F0F0Fu),
                              (int32_t)(kv[bt].y & 0x0F0F0F0Fu), (int32_t)((kv[bt].y >> 4) & 0x0F0F0F0Fu)};
          acc[bt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[0], b0, i32x4_t{0, 0, 0, 0}, 0, 0, 0);
        }
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          const i32x4_t b1 = {(int32_t)(kv[bt].z & 0x0F0F0F0Fu), (int32_t)((kv[bt].z >> 4) & 0x0F0F0F0Fu),
                              (int32_t)(kv[bt].w & 0x0F0F0F0Fu), (int32_t)((kv[bt].w >> 4) & 0x0F0F0F0Fu)};
          acc[bt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[1], b1, acc[bt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const int i = 16 * (q4 + bt) + n16;
        const float raw = __builtin_fmaf((float)acc[bt][3], 16777216.0f,
                                         __builtin_fmaf((float)acc[bt][2], 65536.0f,
                                                        __builtin_fmaf((float)acc[bt][1], 256.0f, (float)acc[bt][0])));
        const float sco = __builtin_fmaf(f16_value(s_sr[0][i][wave]) * raw, rs, f16_value(s_sr[1][i][wave]) * zq);
        scv[q4 + bt] = i < nv ? sco : -INFINITY;
        mw = fmaxf(mw, scv[q4 + bt]);
      }
    }
    mw = row_max16(mw);
    vsm = row_max16(vsm);
    vsm = fmaxf(fmaxf(row_value(vsm, 0), row_value(vsm, 1)), fmaxf(row_value(vsm, 2), row_value(vsm, 3)));
    int ex;
    (void)__builtin_frexpf(vsm, &ex);
    const int Ew = 27 - ex;
    const float Mnew = fmaxf(Mrun, mw);
    const bool grow = __builtin_amdgcn_ballot_w64(Mnew > Mrun) != 0;
    if (grow || first || Ew < Ecur || since >= 1024) {  // wave-uniform
      flush(__builtin_amdgcn_exp2f(Mrun - Mnew));
      Mrun = Mnew;
      Ecur = Ew;
      since = 0;
      first = false;
    }
    ++since;
    // pass 1.5: weight integers of the lane's slots
    const float Mk = Mrun - (float)Ecur;
#pragma unroll
    for (int bk = 0; bk < WN / 16; ++bk) {
      const int i = 16 * bk + n16;
      const float pe = __builtin_amdgcn_exp2f(scv[bk] - Mk);
      Lp += pe;
      Zp = __builtin_fmaf(pe, f16_value(s_sr[3][i][wave]), Zp);
      sn[g * SR + i] = weight_digits((uint32_t)__builtin_fmaf(pe, f16_value(s_sr[2][i][wave]), 0.5f));
    }
    wave_lds_sync();
    // pass 2: value product per 64-slot group
#pragma unroll
    for (int q4 = 0; q4 < WN / 16; q4 += 4) {
      uint32_t D[4], X[4][4];  // X[b][bt]: byte j = code byte b of the lane's channels in slot j of block bt
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const int i0 = 16 * (q4 + bt) + 4 * g;
        const u32x4_t nw = *reinterpret_cast<const u32x4_t*>(&sn[qm * SR + i0]);
        D[bt] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(nw.w, nw.z, dsel), __builtin_amdgcn_perm(nw.y, nw.x, dsel),
                                      0x05040100u);  // byte j: digit qs of slot i0 + j
        if constexpr (BITS == 2) {
          const uint8_t* p0 = s_vc + i0 * kRowB + CB * wave + 4 * (n16 >> 1);
          const uint32_t d0 = *reinterpret_cast<const uint32_t*>(p0), d1 = *reinterpret_cast<const uint32_t*>(p0 + kRowB);
          const uint32_t d2 = *reinterpret_cast<const uint32_t*>(p0 + 2 * kRowB),
                         d3 = *reinterpret_cast<const uint32_t*>(p0 + 3 * kRowB);
          const uint32_t lw = __builtin_amdgcn_perm(d1, d0, vsel), hw = __builtin_amdgcn_perm(d3, d2, vsel);
          X[0][bt] = __builtin_amdgcn_perm(hw, lw, 0x06040200u);
          X[1][bt] = __builtin_amdgcn_perm(hw, lw, 0x07050301u);
        } else {  // 4-bit: the lane's 4 code bytes (channels 8 n16 .. +7) of 4 slots, transposed
          const uint8_t* p0 = s_vc + i0 * kRowB + CB * wave + 4 * n16;
          const uint32_t d0 = *reinterpret_cast<const uint32_t*>(p0), d1 = *reinterpret_cast<const uint32_t*>(p0 + kRowB);
          const uint32_t d2 = *reinterpret_cast<const uint32_t*>(p0 + 2 * kRowB),
                         d3 = *reinterpret_cast<const uint32_t*>(p0 + 3 * kRowB);
          const uint32_t t01 = __builtin_amdgcn_perm(d1, d0, 0x05010400u), t23 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
          const uint32_t u01 = __builtin_amdgcn_perm(d1, d0, 0x07030602u), u23 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
          X[0][bt] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
          X[1][bt] = __builtin_amdgcn_perm(t23, t01, 0x07060302u);
          X[2][bt] = __builtin_amdgcn_perm(u23, u01, 0x05040100u);
          X[3][bt] = __builtin_amdgcn_perm(u23, u01, 0x07060302u);
        }
      }
      const i32x4_t bop = {(int32_t)D[0], (int32_t)D[1], (int32_t)D[2], (int32_t)D[3]};
      if constexpr (BITS == 2) {
        value_product(X[0], X[1], bop, cv);
      } else {  // product 2 b + c: channel 8 n16 + 2 b + c, c = low / high nibble of code byte b
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const i32x4_t lo = {(int32_t)(X[bb][0] & 0x0F0F0F0Fu), (int32_t)(X[bb][1] & 0x0F0F0F0Fu),
                              (int32_t)(X[bb][2] & 0x0F0F0F0Fu), (int32_t)(X[bb][3] & 0x0F0F0F0Fu)};
          const i32x4_t hi = {(int32_t)((X[bb][0] >> 4) & 0x0F0F0F0Fu), (int32_t)((X[bb][1] >> 4) & 0x0F0F0F0Fu),
                              (int32_t)((X[bb][2] >> 4) & 0x0F0F0F0Fu), (int32_t)((X[bb][3] >> 4) & 0x0F0F0F0Fu)};
          cv[2 * bb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(lo, bop, cv[2 * bb], 0, 0, 0);
          cv[2 * bb + 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(hi, bop, cv[2 * bb + 1], 0, 0, 0);
        }
      }
    }
  };
  for (int64_t wt0 = t_begin; wt0 < t_end; wt0 += SW) window(wt0, RA);
  if (t_begin < t_end) flush(1.0f);
  Lf = row_sum16(Lf);
  Zf = row_sum16(Zf);
  const float Lm = __shfl(Lf, 16 * qm), Zm = __shfl(Zf, 16 * qm), Mm = __shfl(Mrun, 16 * qm);
  if (qm < QG) {
    float* pb = a.part + ((r * a.q_heads + h * QG + qm) * a.n_chunks + c) * kAttendPart;
#pragma unroll
    for (int b = 0; b < 8; ++b) pb[32 * g + 8 * qs + b] = fo[b] + Zm;
    if (qs == 0 && g == 0) {
      pb[128] = (t_begin < t_end) ? Mm * 0.6931471805599453f : -INFINITY;
      pb[129] = Lm;
    }
  }
}

// Merge the chunks of each (row, query head), rotate back, add the sink slots, normalise.
__global__ void __launch_bounds__(256) attend_combine(const AttendArgs a) {
  __shared__ float s_out[4][128];
  __shared__ float s_sc[4][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= a.rows * a.q_heads) return;  // wave-uniform; no block barrier in this kernel
  const int64_t r = w / a.q_heads, m = w % a.q_heads;
  const int64_t h = m / (a.q_heads / a.heads);
  int64_t len = a.tokens;
  if (a.lengths) {
    const int64_t n = a.lengths[r];
    len = n < 0 ? 0 : (n > a.tokens ? a.tokens : n);
  }
  const float* pb = a.part + w * (int64_t)a.n_chunks * kAttendPart;
  float M = -INFINITY;
  for (int c = 0; c < a.n_chunks; ++c) M = fmaxf(M, pb[c * kAttendPart + 128]);
  float L = 0.0f, a0 = 0.0f, a1 = 0.0f;
  for (int c = 0; c < a.n_chunks; ++c) {
    const float mc = pb[c * kAttendPart + 128];
    const float f = (mc == -INFINITY) ? 0.0f : __expf(mc - M);
    L = __builtin_fmaf(f, pb[c * kAttendPart + 129], L);
    a0 = __builtin_fmaf(f, pb[c * kAttendPart + lane], a0);
    a1 = __builtin_fmaf(f, pb[c * kAttendPart + lane + 64], a1);
  }
  // back from the rotated domain: z = M acc, then out[perm[j]] = z[j]
  float* so = s_out[wave];
  float z0 = a0, z1 = a1;
  fwht128_wave(z0, z1, lane);
  so[a.use_perm_v ? a.perm_v[lane] : lane] = z0 * kInvSqrt128;
  so[a.use_perm_v ? a.perm_v[lane + 64] : lane + 64] = z1 * kInvSqrt128;
  wave_lds_sync();
  const float y0 = so[lane], y1 = so[lane + 64];
  // sink slots: raw query against the fp16 keys, fp16 values, unrotated
  const int nsk = (int)min((int64_t)a.n_sink, len);
  const float* qr = a.q + w * 128;
  const float q0 = qr[lane], q1 = qr[lane + 64];
  float Mp = M;
  // four sink slots at a time: their cross-lane sums interleave instead of queueing one after another
  for (int t0 = 0; t0 < nsk; t0 += 4) {
    float d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + j < nsk ? t0 + j : t0;  // (a repeated slot past the end is not used)
      const uint16_t* kk = a.k_sink + ((r * a.n_sink + t) * a.heads + h) * 128;
      d[j] = __builtin_fmaf(q0, f16_value(kk[lane]), q1 * f16_value(kk[lane + 64]));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
#pragma unroll
      for (int j = 0; j < 4; ++j) d[j] += __shfl_xor(d[j], o);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (t0 + j < nsk) {
        const float st = d[j] * a.scale;
        if (lane == 0) s_sc[wave][t0 + j] = st;
        Mp = fmaxf(Mp, st);
      }
    }
  }
  wave_lds_sync();
  const float f = (M == -INFINITY) ? 0.0f : __expf(M - Mp);
  float n0 = f * y0, n1 = f * y1, den = f * L;
  for (int t = 0; t < nsk; ++t) {
    const float e = __expf(s_sc[wave][t] - Mp);
    const uint16_t* vv = a.v_sink + ((r * a.n_sink + t) * a.heads + h) * 128;
    n0 = __builtin_fmaf(e, f16_value(vv[lane]), n0);
    n1 = __builtin_fmaf(e, f16_value(vv[lane + 64]), n1);
    den += e;
  }
  float* out = a.out + w * 128;
  out[lane] = den > 0.0f ? n0 / den : 0.0f;
  out[lane + 64] = den > 0.0f ? n1 / den : 0.0f;
}

// ---------------------------------------------------------------------------
// DECODE-STEP ATTENTION, GENERAL PASS: head_dim 128 or 256, Walsh-Hadamard or no rotation,
// min-max codes of 2, 3 or 4 bits for K and V each (each its own group size), 1 to 8 query
// heads per KV head, and a cache whose slot 0 holds position pos_offset (the sink slots are
// the positions below n_sink).  The same three passes in the rotated domain as above; the
// scores and value sums run on the vector ALUs.
// ---------------------------------------------------------------------------

// Unnormalised Walsh-Hadamard transform (Sylvester order) of D values held by a wave as
// u[k] = x[lane + 64 k]: index bits 6.. inside the lane, bits 0..5 across lanes.
template <int D>
__device__ __forceinline__ void fwht_wave(float (&u)[D / 64], int lane) {
  constexpr int K = D / 64;
#pragma unroll
  for (int hb = 1; hb < K; hb <<= 1)
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (!(k & hb)) {
        const float x = u[k], y = u[k + hb];
        u[k] = x + y;
        u[k + hb] = x - y;
      }
#pragma unroll
  for (int bit = 1; bit < 64; bit <<= 1)
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const float p = __shfl_xor(u[k], bit);
      u[k] = (lane & bit) ? p - u[k] : u[k] + p;
    }
}

// rotated queries M P q (M = H / sqrt(D), or the identity without rotation): one wave per
// (row, query head)
template <int D>
__global__ void __launch_bounds__(256) attend_rotate_q_gen(const AttendArgs a) {
  constexpr int K = D / 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= a.rows * a.q_heads) return;  // wave-uniform; no barrier in this kernel
  const float* q = a.q + w * D;
  float u[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int c = lane + 64 * k;
    u[k] = q[a.use_perm_k ? a.perm_k[c] : c];  // (P q)[c] = q[perm[c]]
  }
  float nc = 1.0f;
  if (a.rot) {
    fwht_wave<D>(u, lane);
    nc = (float)(1.0 / __builtin_sqrt((double)D));
  }
#pragma unroll
  for (int k = 0; k < K; ++k) a.qrot[w * D + lane + 64 * k] = u[k] * nc;
}

// The 16 codes of a lane (channels 16 l .. 16 l + 15 of a vector, 2 BITS bytes at byte
// 2 BITS l of its record).  3-bit records put a lane's 6 bytes on a 2-byte boundary when l
// is odd: the two aligned words that cover them (inside the record: 6 l + 6 <= 6 l' + 8 for
// l' = l rounded down to even, and the record ends at a multiple of 12 bytes from l' = 0)
// are shifted down by 16 bits.
template <int BITS>
struct SlotCodes {
  uint32_t w[BITS == 2 ? 1 : 2];
};
template <int BITS>
__device__ __forceinline__ uint32_t slot_code_offset(int l) {  // the lane's first word in its record
  return BITS == 2 ? 4u * (uint32_t)l : (BITS == 4 ? 8u * (uint32_t)l : (uint32_t)((6 * l) & ~3));
}
// the lane's words at byte off of the descriptor (reads past its end give zeros)
template <int BITS>
__device__ __forceinline__ void load_slot_codes(buf_t b, uint32_t off, SlotCodes<BITS>& c) {
  if constexpr (BITS == 2) {
    c.w[0] = __builtin_amdgcn_raw_buffer_load_b32(b, off, 0, 0);
  } else {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(b, off, 0, 0);  // 4-byte aligned
    c.w[0] = v.x;
    c.w[1] = v.y;
  }
}
// codes to floats (for 3 bits the word pair is first shifted into place, see above)
template <int BITS>
__device__ __forceinline__ void slot_code_floats(SlotCodes<BITS> c, int l, float (&code)[16]) {
  if constexpr (BITS == 3) {
    const uint32_t sh = (uint32_t)(l & 1) * 16u;
    const uint32_t lo = __builtin_amdgcn_alignbit(c.w[1], c.w[0], sh), hi = c.w[1] >> sh;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int bit = 3 * i;
      uint32_t v;
      if (bit + 3 <= 32) v = lo >> bit;
      else if (bit >= 32) v = hi >> (bit - 32);
      else v = (lo >> bit) | (hi << (32 - bit));
      code[i] = (float)(v & 7u);
    }
  } else {
    // spread each word's codes over bytes, then one byte-to-float conversion per code
    constexpr int PER = 32 / BITS, SPR = 8 / BITS;
    constexpr uint32_t BM = (BITS == 2) ? 0x03030303u : 0x0F0F0F0Fu;
#pragma unroll
    for (int j = 0; j < BITS / 2; ++j)
#pragma unroll
      for (int k = 0; k < SPR; ++k) {
        uint32_t e = (c.w[j] >> (BITS * k)) & BM;  // byte b holds code SPR * b + k of word j
        asm volatile("" : "+v"(e));
#pragma unroll
        for (int b = 0; b < 4; ++b) code[PER * j + SPR * b + k] = (float)((e >> (8 * b)) & 0xffu);
      }
  }
}

// Partial pass: one wave per (row, KV head, chunk of slots).  Lane (tk, l) = (lane / LPS,
// lane % LPS), LPS = D / 16 lanes per slot, holds channels 16 l .. 16 l + 15 of slot tk of
// each step of 64 / LPS slots; the LPS lanes of a slot reduce its scores, and each slot keeps
// its own running maximum, denominator and rotated-domain sums until the wave merges them.
template <int D, int KB, int VB, int QG>
__global__ void __launch_bounds__(256) attend_partial_gen(const AttendArgs a) {
  constexpr int LPS = D / 16, SPS = 64 / LPS;
  constexpr int KCB = D * KB / 8, VCB = D * VB / 8;  // code bytes per vector
  constexpr int PS = D + 2;                          // floats per partial
  __shared__ __attribute__((aligned(16))) float s_qv[4][QG * D];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= a.rows * a.heads * a.n_chunks) return;  // wave-uniform; no block barrier follows
  const int64_t c = w % a.n_chunks, rh = w / a.n_chunks, h = rh % a.heads, r = rh / a.heads;
  const int tk = lane / LPS, l = lane % LPS;
  int64_t len = a.tokens;
  if (a.lengths) {
    const int64_t n = a.lengths[r];
    len = n < 0 ? 0 : (n > a.tokens ? a.tokens : n);
  }
  const int64_t t_begin = max(c * (int64_t)a.chunk, (int64_t)a.sink_slots);
  const int64_t t_end = min((c + 1) * (int64_t)a.chunk, len);
  const int64_t kng = D >> a.group_log2, vng = D >> a.v_group_log2;
  const int kg = (16 * l) >> a.group_log2, vg = (16 * l) >> a.v_group_log2;  // groups of >= 32

  float sl[QG];
  {
    const float* src = a.qrot + (r * a.q_heads + h * QG) * D;
    for (int i = lane; i < QG * D; i += 64) s_qv[wave][i] = src[i];
    wave_lds_sync();
  }
  const uint32_t qaddr = lds_addr(&s_qv[wave][16 * l]);
#pragma unroll
  for (int m = 0; m < QG; ++m) {
    sl[m] = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4_t v = lds_ld4(qaddr + 4u * D * m + 16u * k);
      sl[m] += (__uint_as_float(v.x) + __uint_as_float(v.y)) + (__uint_as_float(v.z) + __uint_as_float(v.w));
    }
  }
  float mx[QG], ls[QG], zs[QG], acc[QG][16];
#pragma unroll
  for (int m = 0; m < QG; ++m) {
    mx[m] = -INFINITY;
    ls[m] = 0.0f;
    zs[m] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[m][i] = 0.0f;
  }
  struct Slot {
    SlotCodes<KB> k;
    SlotCodes<VB> v;
    uint32_t ks, kz, vs, vz;  // fp16 bits of the lane's group scale and zero
  };
  // The lane's slot of step t0, through descriptors based at (row r, slot t0, head h) that end
  // with the record of (slot t_end - 1, head h): the per-step address arithmetic is scalar, the
  // lane's offsets are fixed (below 8 slots * 32768 heads * 128 bytes: heads <= 32768 on the
  // host), and lanes past the chunk's end read zeros (their slots are masked afterwards).
  const int64_t vb = r * a.tokens * a.heads + h;  // vector (row r, slot 0, head h)
  const uint32_t th = (uint32_t)tk * (uint32_t)a.heads;
  const uint32_t kco = th * KCB + slot_code_offset<KB>(l), vco = th * VCB + slot_code_offset<VB>(l);
  const uint32_t kso = 2u * (th * (uint32_t)kng + (uint32_t)kg), vso = 2u * (th * (uint32_t)vng + (uint32_t)vg);
  auto load = [&](int64_t t0, Slot& s) __attribute__((always_inline)) {
    const int64_t v0 = vb + t0 * a.heads;  // vector (row r, slot t0, head h)
    // vectors up to (row r, slot min(t_end - 1, t0 + SPS - 1), head h), none past the chunk's end,
    // in 32-bit scalar arithmetic (slots < 2^31; at most SPS * heads vectors, below 2^18)
    const int32_t rem = (int32_t)(t_end - 1 - t0);
    const uint32_t nv = rem < 0 ? 0u : (uint32_t)min(rem, SPS - 1) * (uint32_t)a.heads + 1u;
    load_slot_codes<KB>(make_buf_item(a.k_codes + v0 * KCB, nv * KCB), kco, s.k);
    load_slot_codes<VB>(make_buf_item(a.v_codes + v0 * VCB, nv * VCB), vco, s.v);
    const uint32_t kgb = 2u * nv * (uint32_t)kng, vgb = 2u * nv * (uint32_t)vng;
    s.ks = __builtin_amdgcn_raw_buffer_load_b16(make_buf_item(a.k_scale + v0 * kng, kgb), kso, 0, 0);
    s.kz = __builtin_amdgcn_raw_buffer_load_b16(make_buf_item(a.k_zero + v0 * kng, kgb), kso, 0, 0);
    s.vs = __builtin_amdgcn_raw_buffer_load_b16(make_buf_item(a.v_scale + v0 * vng, vgb), vso, 0, 0);
    s.vz = __builtin_amdgcn_raw_buffer_load_b16(make_buf_item(a.v_zero + v0 * vng, vgb), vso, 0, 0);
  };

  // loads in flight two steps ahead: measured 13 % faster than one at the wide-head cache, and
  // the third slot's registers leave every instance at its occupancy
  const int32_t vlim = (int32_t)(t_end - tk);  // the lane's slot of step t0 exists iff t0 < vlim
  if (t_begin < t_end) {
    Slot cur, nx1, nx2;
    load(t_begin, cur);
    if (t_begin + SPS < t_end) load(t_begin + SPS, nx1);
    for (int64_t t0 = t_begin; t0 < t_end; t0 += SPS) {
      if (t0 + 2 * SPS < t_end) load(t0 + 2 * SPS, nx2);  // wave-uniform
      const bool valid = (int32_t)t0 < vlim;
      float code[16];
      slot_code_floats<KB>(cur.k, l, code);
      const float ks = f16_value(cur.ks), kz = f16_value(cur.kz);
      float s[QG];
      uint32_t qa = qaddr;
      asm volatile("" : "+v"(qa));  // read the slices here, each step (not hoisted into registers)
#pragma unroll
      for (int m = 0; m < QG; ++m) {
        float d = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const u32x4_t v = lds_ld4(qa + 4u * D * m + 16u * k);
          d = __builtin_fmaf(__uint_as_float(v.x), code[4 * k + 0], d);
          d = __builtin_fmaf(__uint_as_float(v.y), code[4 * k + 1], d);
          d = __builtin_fmaf(__uint_as_float(v.z), code[4 * k + 2], d);
          d = __builtin_fmaf(__uint_as_float(v.w), code[4 * k + 3], d);
        }
        float part = __builtin_fmaf(ks, d, kz * sl[m]);  // q~ . (zero + code * scale) over 16 channels
        part = add_x1(part);
        part = add_x2(part);
        part = add_half_mirror(part);
        if constexpr (LPS == 16) part = add_row_mirror(part);
        s[m] = valid ? part * a.scale : -INFINITY;
      }
      bool grow = false;
      float mn[QG];
#pragma unroll
      for (int m = 0; m < QG; ++m) {
        mn[m] = fmaxf(mx[m], s[m]);
        grow |= mn[m] > mx[m];
      }
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
        for (int m = 0; m < QG; ++m) {
          const float corr = (mn[m] > mx[m]) ? __expf(mx[m] - mn[m]) : 1.0f;
          ls[m] *= corr;
          zs[m] *= corr;
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[m][i] *= corr;
          mx[m] = mn[m];
        }
      }
      slot_code_floats<VB>(cur.v, l, code);
      const float vs = f16_value(cur.vs), vz = f16_value(cur.vz);
#pragma unroll
      for (int m = 0; m < QG; ++m) {
        const float p = valid ? __expf(s[m] - mx[m]) : 0.0f;
        ls[m] += p;
        zs[m] = __builtin_fmaf(p, vz, zs[m]);
        const float ps = p * vs;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][i] = __builtin_fmaf(ps, code[i], acc[m][i]);
      }
      cur = nx1;
      nx1 = nx2;
    }
  }
  // merge the wave's slots (lanes xor LPS, 2 LPS, ...) and write the chunk's partial
#pragma unroll
  for (int m = 0; m < QG; ++m) {
    float M = mx[m];
#pragma unroll
    for (int o = LPS; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float f = (mx[m] == -INFINITY) ? 0.0f : __expf(mx[m] - M);
    float L = ls[m] * f;
#pragma unroll
    for (int o = LPS; o < 64; o <<= 1) L += __shfl_xor(L, o);
    float* pb = a.part + ((r * a.q_heads + h * QG + m) * a.n_chunks + c) * PS;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = (acc[m][i] + zs[m]) * f;
#pragma unroll
      for (int o = LPS; o < 64; o <<= 1) v += __shfl_xor(v, o);
      if (tk == 0) pb[16 * l + i] = v;
    }
    if (lane == 0) {
      pb[D] = M;
      pb[D + 1] = L;
    }
  }
}

// Merge of the chunks, rotation back (z = M acc, out[perm[j]] = z[j]), the sink slots (raw
// query against the fp16 keys of the sink plane, entry pos_offset + slot) and the
// normalisation: one wave per (row, query head).
template <int D>
__global__ void __launch_bounds__(256) attend_combine_gen(const AttendArgs a) {
  constexpr int K = D / 64, PS = D + 2;
  __shared__ float s_out[4][D];
  __shared__ float s_sc[4][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= a.rows * a.q_heads) return;  // wave-uniform; no block barrier in this kernel
  const int64_t r = w / a.q_heads, m = w % a.q_heads;
  const int64_t h = m / (a.q_heads / a.heads);
  int64_t len = a.tokens;
  if (a.lengths) {
    const int64_t n = a.lengths[r];
    len = n < 0 ? 0 : (n > a.tokens ? a.tokens : n);
  }
  const float* pb = a.part + w * (int64_t)a.n_chunks * PS;
  float M = -INFINITY;  // the chunks' maxima read by the lanes in parallel, then a wave maximum
  for (int c = lane; c < a.n_chunks; c += 64) M = fmaxf(M, pb[c * PS + D]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
  float L = 0.0f, acc[K];
#pragma unroll
  for (int k = 0; k < K; ++k) acc[k] = 0.0f;
#pragma unroll 4
  for (int c = 0; c < a.n_chunks; ++c) {
    const float mc = pb[c * PS + D];
    const float f = (mc == -INFINITY) ? 0.0f : __expf(mc - M);
    L = __builtin_fmaf(f, pb[c * PS + D + 1], L);
#pragma unroll
    for (int k = 0; k < K; ++k) acc[k] = __builtin_fmaf(f, pb[c * PS + lane + 64 * k], acc[k]);
  }
  float* so = s_out[wave];
  float nc = 1.0f;
  if (a.rot) {
    fwht_wave<D>(acc, lane);
    nc = (float)(1.0 / __builtin_sqrt((double)D));
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int j = lane + 64 * k;
    so[a.use_perm_v ? a.perm_v[j] : j] = acc[k] * nc;
  }
  wave_lds_sync();
  float y[K];
#pragma unroll
  for (int k = 0; k < K; ++k) y[k] = so[lane + 64 * k];
  const int nsk = (int)min((int64_t)a.sink_slots, len);
  const float* qr = a.q + w * D;
  float qv[K];
#pragma unroll
  for (int k = 0; k < K; ++k) qv[k] = qr[lane + 64 * k];
  float Mp = M;
  for (int t = 0; t < nsk; ++t) {
    const uint16_t* kk = a.k_sink + ((r * a.n_sink + a.sink_base + t) * a.heads + h) * D;
    float d = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) d = __builtin_fmaf(qv[k], f16_value(kk[lane + 64 * k]), d);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) d += __shfl_xor(d, o);
    const float st = d * a.scale;
    if (lane == 0) s_sc[wave][t] = st;
    Mp = fmaxf(Mp, st);
  }
  wave_lds_sync();
  const float f = (M == -INFINITY) ? 0.0f : __expf(M - Mp);
  float n[K], den = f * L;
#pragma unroll
  for (int k = 0; k < K; ++k) n[k] = f * y[k];
  for (int t = 0; t < nsk; ++t) {
    const float e = __expf(s_sc[wave][t] - Mp);
    const uint16_t* vv = a.v_sink + ((r * a.n_sink + a.sink_base + t) * a.heads + h) * D;
#pragma unroll
    for (int k = 0; k < K; ++k) n[k] = __builtin_fmaf(e, f16_value(vv[lane + 64 * k]), n[k]);
    den += e;
  }
  float* out = a.out + w * D;
#pragma unroll
  for (int k = 0; k < K; ++k) out[lane + 64 * k] = den > 0.0f ? n[k] / den : 0.0f;
}

// ---------------------------------------------------------------------------
// launch dispatch
// ---------------------------------------------------------------------------
// Grid of a launch: one wave per task (len rows of one tile, or len tiles of one row).
int plan_grid(CodecArgs& b, bool tiles_of_a_row, int len, unsigned& nb) {
  b.task_len = len;
  b.n_tblk = (b.n_tiles + len - 1) / len;
  b.div_task = make_fastdiv((uint32_t)(tiles_of_a_row ? b.n_tblk : b.n_tiles));
  const int64_t tasks = tiles_of_a_row ? b.rows * b.n_tblk : b.n_tiles * ((b.rows + len - 1) / len);
  const int64_t blocks = (tasks + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks * kWavesPerBlock > 0x7fffffff) return (int)hipErrorInvalidConfiguration;  // wave ids < 2^31
  nb = (unsigned)blocks;
  return 0;
}

template <int DT, int D, int BITS, int ROT, int QUANT, int RT, int PT, int GBT, int AP = 0>
int launch_enc_t(const CodecArgs& a, hipStream_t s) {
  if (a.n_items == 0) return 0;
  constexpr int VPW = Geo<D>::VPW;
  CodecArgs b = a;
  // tokens a tile of VPW columns can span: floor((h0 + VPW - 1) / heads) + 1, h0 < heads
  b.trig_rows = (int32_t)std::min<int64_t>(VPW, (a.heads - 1 + VPW - 1) / a.heads + 1);
  // Rows per task, the fastest measured on MI355X at the Llama-3 cache shape: with RoPE a
  // wave's cos/sin table serves 8 rows; with only a permutation its gather addresses
  // serve 2; otherwise one item per wave.
  const size_t lds =
      (size_t)kWavesPerBlock * enc_wave_bytes<D>(a.use_perm != 0 || ROT == ROT_ROTOR, a.rope != 0, b.trig_rows);
  unsigned nb = 0;
  if (int e = plan_grid(b, false, AP ? 1 : (a.rope ? 8 : (a.use_perm ? 2 : 1)), nb)) return e;
  hipLaunchKernelGGL((encode_kernel<DT, D, BITS, ROT, QUANT, RT, PT, GBT, AP>), dim3(nb), dim3(64 * kWavesPerBlock),
                     lds, s, b);
  if (hipError_t e = hipGetLastError()) return (int)e;
  if constexpr (AP) return 0;  // the append kernel writes sink positions itself
  if (const unsigned ns = sink_blocks(a, Geo<D>::LV)) {
    hipLaunchKernelGGL((encode_sink_kernel<DT, D, BITS, QUANT>), dim3(ns), dim3(64 * kWavesPerBlock), 0, s, b);
    return (int)hipGetLastError();
  }
  return 0;
}

template <int ODT, int D, int BITS, int ROT, int QUANT, int PT>
int launch_dec_t(const CodecArgs& a, hipStream_t s) {
  if (a.n_items == 0) return 0;
  const size_t lds = (size_t)kWavesPerBlock * Geo<D>::VPW *
                     (dec_row_bytes<D, ODT>() + (ROT == ROT_ROTOR ? D * 4 + 16 : 0));
  CodecArgs b = a;
  unsigned nb = 0;
  // one tile per wave (a 4 KiB output run at d = 128, bf16; measured 10 % faster than 4 tiles
  // at the Llama-3 cache shape: short runs per wave stream writes faster), 8 tiles with the
  // permutation (1, 2 and 4 measured 36 %, 14 % and 2 % slower there)
  if (int e = plan_grid(b, true, PT != 0 ? 8 : 1, nb)) return e;
  hipLaunchKernelGGL((decode_kernel<ODT, D, BITS, ROT, QUANT, PT>), dim3(nb), dim3(64 * kWavesPerBlock), lds, s,
                     b);
  if (hipError_t e = hipGetLastError()) return (int)e;
  if (const unsigned ns = sink_blocks(a, Geo<D>::LV)) {
    hipLaunchKernelGGL((decode_sink_kernel<ODT, D>), dim3(ns), dim3(64 * kWavesPerBlock), 0, s, b);
    return (int)hipGetLastError();
  }
  return 0;
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
    // append: features read from the arguments (a launch of a few thousand vectors)
    if (a.row_pos) return launch_enc_t<DT, D, BITS, ROT, QUANT, -1, -1, -1, 1>(a, s);
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
    case ROT_ROTOR: return pick_quant<ENC, DT, D, BITS, ROT_ROTOR>(quant, a, s);
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
#if KVQ_UNIT == 12 || KVQ_UNIT == -1
namespace {
template <int BITS, int QG>
int launch_attend_t(const AttendArgs& a, hipStream_t s) {
  const int64_t nq = a.rows * a.q_heads;
  const int64_t np = a.rows * a.heads * a.n_chunks;
  if (nq == 0) return 0;
  if ((np + 3) / 4 > 0x7fffffff || (nq + 3) / 4 > 0x7fffffff) return (int)hipErrorInvalidConfiguration;
  const uintptr_t al4 = (uintptr_t)a.k_codes | (uintptr_t)a.v_codes | (uintptr_t)a.k_scale | (uintptr_t)a.k_zero |
                        (uintptr_t)a.v_scale | (uintptr_t)a.v_zero;
  // the block-cooperative pass rotates its queries itself; the others read them from the workspace
  const bool blk = a.group_log2 == 7 && a.heads % 4 == 0 && (al4 & 7) == 0 && (BITS == 4 || BITS == 2);
  if (!blk) {
    hipLaunchKernelGGL(attend_rotate_q, dim3((unsigned)((nq + 3) / 4)), dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError()) return (int)e;
  }
  if (BITS == 4 && a.group_log2 == 7 && a.heads % 4 == 0 && (al4 & 7) == 0) {
    const int64_t nb = ((np + 3) / 4 + 15) / 16 * 16;  // whole groups of 16 blocks (XCD-aware order)
    if (nb > 0x7fffffff) return (int)hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attend_partial_mma_blk<4, QG>), dim3((unsigned)nb), dim3(256), 0, s, a);
  } else if (BITS == 2 && a.group_log2 == 7 && ((uintptr_t)a.k_codes & 7) == 0 && ((uintptr_t)a.v_codes & 1) == 0) {
    // whole groups of 16 blocks, so the XCD-aware order maps the blocks onto every task
    const int64_t nb = ((np + 3) / 4 + 15) / 16 * 16;
    if (nb > 0x7fffffff) return (int)hipErrorInvalidConfiguration;
    const uintptr_t al = (uintptr_t)a.k_codes | (uintptr_t)a.v_codes | (uintptr_t)a.k_scale | (uintptr_t)a.k_zero |
                         (uintptr_t)a.v_scale | (uintptr_t)a.v_zero;
    if (a.heads % 4 == 0 && (al & 7) == 0)
      hipLaunchKernelGGL((attend_partial_mma_blk<2, QG>), dim3((unsigned)nb), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((attend_partial_mma<QG>), dim3((unsigned)nb), dim3(256), 0, s, a);
  } else
    hipLaunchKernelGGL((attend_partial<BITS, QG>), dim3((unsigned)((np + 3) / 4)), dim3(256), 0, s, a);
  if (hipError_t e = hipGetLastError()) return (int)e;
  hipLaunchKernelGGL(attend_combine, dim3((unsigned)((nq + 3) / 4)), dim3(256), 0, s, a);
  return (int)hipGetLastError();
}
}  // namespace
// Workspace of kvq_attend_noalloc: callers that cannot allocate get the rotated queries and the
// partials here instead of in a buffer of their own.  Host code never passes the array's name to
// a kernel (on the host it names a stand-in, not device memory): it passes the device address
// looked up below, one per device.
static __device__ __attribute__((aligned(256))) unsigned char scratch[kAttendScratchBytes];

int attend_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

int launch_attend(int bits, int qg, const AttendArgs& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (bits == 2) {
    if (qg == 1) return launch_attend_t<2, 1>(a, s);
    if (qg == 2) return launch_attend_t<2, 2>(a, s);
    return launch_attend_t<2, 4>(a, s);
  }
  if (qg == 1) return launch_attend_t<4, 1>(a, s);
  if (qg == 2) return launch_attend_t<4, 2>(a, s);
  return launch_attend_t<4, 4>(a, s);
}
#endif

#if (KVQ_UNIT >= 14 && KVQ_UNIT <= 19) || KVQ_UNIT == -1
namespace {
template <int D, int KB, int VB, int QG>
int launch_attend_gen_t(const AttendArgs& a, hipStream_t s) {
  const int64_t nq = a.rows * a.q_heads;
  const int64_t np = a.rows * a.heads * a.n_chunks;
  if (nq == 0) return 0;
  if ((np + 3) / 4 > 0x7fffffff || (nq + 3) / 4 > 0x7fffffff) return (int)hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attend_rotate_q_gen<D>), dim3((unsigned)((nq + 3) / 4)), dim3(256), 0, s, a);
  if (hipError_t e = hipGetLastError()) return (int)e;
  hipLaunchKernelGGL((attend_partial_gen<D, KB, VB, QG>), dim3((unsigned)((np + 3) / 4)), dim3(256), 0, s, a);
  if (hipError_t e = hipGetLastError()) return (int)e;
  hipLaunchKernelGGL((attend_combine_gen<D>), dim3((unsigned)((nq + 3) / 4)), dim3(256), 0, s, a);
  return (int)hipGetLastError();
}
template <int D, int KB, int VB>
int pick_attend_gen_qg(int qg, const AttendArgs& a, hipStream_t s) {
  switch (qg) {
    case 1: return launch_attend_gen_t<D, KB, VB, 1>(a, s);
    case 2: return launch_attend_gen_t<D, KB, VB, 2>(a, s);
    case 4: return launch_attend_gen_t<D, KB, VB, 4>(a, s);
    default: return launch_attend_gen_t<D, KB, VB, 8>(a, s);
  }
}
template <int D, int KB>
int pick_attend_gen(int v_bits, int qg, const AttendArgs& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (v_bits) {
    case 2: return pick_attend_gen_qg<D, KB, 2>(qg, a, s);
    case 3: return pick_attend_gen_qg<D, KB, 3>(qg, a, s);
    default: return pick_attend_gen_qg<D, KB, 4>(qg, a, s);
  }
}
}  // namespace
#endif
#if KVQ_UNIT == 14 || KVQ_UNIT == -1
int launch_attend_gen_d128_k2(int vb, int qg, const AttendArgs& a, void* s) { return pick_attend_gen<128, 2>(vb, qg, a, s); }
#endif
#if KVQ_UNIT == 15 || KVQ_UNIT == -1
int launch_attend_gen_d128_k3(int vb, int qg, const AttendArgs& a, void* s) { return pick_attend_gen<128, 3>(vb, qg, a, s); }
#endif
#if KVQ_UNIT == 16 || KVQ_UNIT == -1
int launch_attend_gen_d128_k4(int vb, int qg, const AttendArgs& a, void* s) { return pick_attend_gen<128, 4>(vb, qg, a, s); }
#endif
#if KVQ_UNIT == 17 || KVQ_UNIT == -1
int launch_attend_gen_d256_k2(int vb, int qg, const AttendArgs& a, void* s) { return pick_attend_gen<256, 2>(vb, qg, a, s); }
#endif
#if KVQ_UNIT == 18 || KVQ_UNIT == -1
int launch_attend_gen_d256_k3(int vb, int qg, const AttendArgs& a, void* s) { return pick_attend_gen<256, 3>(vb, qg, a, s); }
#endif
#if KVQ_UNIT == 19 || KVQ_UNIT == -1
int launch_attend_gen_d256_k4(int vb, int qg, const AttendArgs& a, void* s) { return pick_attend_gen<256, 4>(vb, qg, a, s); }
#endif

#if KVQ_UNIT == 20 || KVQ_UNIT == 21 || KVQ_UNIT == -1
namespace {
// Grid of a dense-rotation pass: one block per CU (the matrix takes 132 KB of its LDS), fewer
// when the tensor has fewer items than 8 per block; blocks stride over the items.
inline unsigned dense_blocks(const CodecArgs& a) {
  const int64_t n_items = (a.rows * a.tokens * a.heads + 15) / 16;
  const int64_t nb = (n_items + kDenseWaves - 1) / kDenseWaves;
  return (unsigned)(nb < 256 ? nb : 256);
}
}  // namespace
#endif
#if KVQ_UNIT == 20 || KVQ_UNIT == -1
namespace {
template <int DT, int BITS, int QUANT>
int launch_enc_dense_t(const CodecArgs& a, hipStream_t s) {
  const unsigned nb = dense_blocks(a);
  if (nb == 0) return 0;
  hipLaunchKernelGGL((encode_dense_kernel<DT, BITS, QUANT>), dim3(nb), dim3(64 * kDenseWaves), 0, s, a);
  if (hipError_t e = hipGetLastError()) return (int)e;
  if (const unsigned ns = sink_blocks(a, Geo<128>::LV)) {
    hipLaunchKernelGGL((encode_sink_kernel<DT, 128, BITS, QUANT>), dim3(ns), dim3(64 * kWavesPerBlock), 0, s, a);
    return (int)hipGetLastError();
  }
  return 0;
}
template <int DT>
int pick_enc_dense(int bits, int quant, const CodecArgs& a, hipStream_t s) {
  if (quant == Q_MINMAX) {
    if (bits == 2) return launch_enc_dense_t<DT, 2, Q_MINMAX>(a, s);
    if (bits == 3) return launch_enc_dense_t<DT, 3, Q_MINMAX>(a, s);
    return launch_enc_dense_t<DT, 4, Q_MINMAX>(a, s);
  }
  if (bits == 2) return launch_enc_dense_t<DT, 2, Q_LLOYD>(a, s);
  if (bits == 3) return launch_enc_dense_t<DT, 3, Q_LLOYD>(a, s);
  return launch_enc_dense_t<DT, 4, Q_LLOYD>(a, s);
}
}  // namespace
int launch_encode_dense(int dtype, int bits, int quant, const CodecArgs& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == DT_F16) return pick_enc_dense<DT_F16>(bits, quant, a, s);
  if (dtype == DT_BF16) return pick_enc_dense<DT_BF16>(bits, quant, a, s);
  return pick_enc_dense<DT_F32>(bits, quant, a, s);
}
#endif
#if KVQ_UNIT == 21 || KVQ_UNIT == -1
namespace {
template <int ODT, int BITS, int QUANT>
int launch_dec_dense_t(const CodecArgs& a, hipStream_t s) {
  const unsigned nb = dense_blocks(a);
  if (nb == 0) return 0;
  hipLaunchKernelGGL((decode_dense_kernel<ODT, BITS, QUANT>), dim3(nb), dim3(64 * kDenseWaves), 0, s, a);
  if (hipError_t e = hipGetLastError()) return (int)e;
  if (const unsigned ns = sink_blocks(a, Geo<128>::LV)) {
    hipLaunchKernelGGL((decode_sink_kernel<ODT, 128>), dim3(ns), dim3(64 * kWavesPerBlock), 0, s, a);
    return (int)hipGetLastError();
  }
  return 0;
}
template <int ODT>
int pick_dec_dense(int bits, int quant, const CodecArgs& a, hipStream_t s) {
  if (quant == Q_MINMAX) {
    if (bits == 2) return launch_dec_dense_t<ODT, 2, Q_MINMAX>(a, s);
    if (bits == 3) return launch_dec_dense_t<ODT, 3, Q_MINMAX>(a, s);
    return launch_dec_dense_t<ODT, 4, Q_MINMAX>(a, s);
  }
  if (bits == 2) return launch_dec_dense_t<ODT, 2, Q_LLOYD>(a, s);
  if (bits == 3) return launch_dec_dense_t<ODT, 3, Q_LLOYD>(a, s);
  return launch_dec_dense_t<ODT, 4, Q_LLOYD>(a, s);
}
}  // namespace
int launch_decode_dense(int out_dtype, int bits, int quant, const CodecArgs& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (out_dtype == DT_F16) return pick_dec_dense<DT_F16>(bits, quant, a, s);
  if (out_dtype == DT_BF16) return pick_dec_dense<DT_BF16>(bits, quant, a, s);
  return pick_dec_dense<DT_F32>(bits, quant, a, s);
}
#endif

#if KVQ_UNIT == 13 || KVQ_UNIT == -1
// ---------------------------------------------------------------------------
// CALIBRATION OF THE ROTATEKV VARIANTS
// ---------------------------------------------------------------------------
// Channel statistics for the outlier-aware permutation: mean |y_c| of the post-RoPE vectors of
// a calibration slice, sink positions left out.  Token norms and a per-row median for the
// activation-based sink detection.  Both read the slice once; neither is on the codec's path.
namespace {
// One wave per (row, run of tpw tokens).  Lane i owns the channel pairs (2i, 2i + 1) (and
// (2i + 128, 2i + 129) at d = 256), so each load instruction of the wave covers one vector's
// bytes contiguously, and the pair's cos/sin is computed once per token for all heads.  A
// token's heads are read in batches of 8 loads issued before any is used; each batch's |y|
// are summed in float32 (8 terms) and added to float64 sums per lane; the per-wave sums go to
// the workspace.
template <int DT, int D>
__global__ void __launch_bounds__(256) channel_stats_kernel(const CalibArgs a) {
  constexpr int NP = D / 128;  // channel pairs per lane
  constexpr int ES = (DT == DT_F32) ? 4 : 2;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= a.n_waves) return;  // wave-uniform; no block barrier in this kernel
  const int64_t nchunk = (a.tokens + a.tpw - 1) / a.tpw;
  const int64_t r = w / nchunk, t0 = (w % nchunk) * a.tpw;
  const int64_t t1 = min(t0 + (int64_t)a.tpw, a.tokens);
  double theta[NP], s0[NP], s1[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    theta[k] = exp2(-(2.0 * (double)(lane + 64 * k) / (double)D) * a.rope_log2_base);
    s0[k] = 0.0;
    s1[k] = 0.0;
  }
  const char* base = reinterpret_cast<const char*>(a.x);
  for (int64_t t = t0; t < t1; ++t) {
    const int64_t pos = a.pos_offset + t;
    if (pos < a.n_sink) continue;  // a sink position (wave-uniform)
    float c[NP], sn[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      c[k] = 1.0f;
      sn[k] = 0.0f;
      if (a.rope) rope_cos_sin(pos, theta[k], &c[k], &sn[k]);
    }
    const char* tb = base + (r * a.sr + t * a.st) * ES;
    for (int64_t h0 = 0; h0 < a.heads; h0 += 8) {  // wave-uniform
      constexpr int EW = (DT == DT_F32) ? 2 : 1;  // 32-bit words per channel pair
      uint32_t wd[8][NP][EW];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // heads past the last read as zeros (|y| = 0 adds nothing); streamed loads, each wave
        // instruction reading whole lines once (measured 6 % faster than temporal ones)
        const buf_t hb = make_buf(tb + (h0 + j) * a.sh * ES, h0 + j < a.heads ? D * ES : 0);
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          const uint32_t off = (uint32_t)(lane + 64 * k) * (4u * EW);
          if constexpr (EW == 2) {
            const u32x2_t xx = __builtin_amdgcn_raw_buffer_load_b64(hb, off, 0, kNT | kSC1);
            wd[j][k][0] = xx.x;
            wd[j][k][EW - 1] = xx.y;
          } else {
            wd[j][k][0] = __builtin_amdgcn_raw_buffer_load_b32(hb, off, 0, kNT | kSC1);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float x0, x1;
          if constexpr (DT == DT_F32) {
            x0 = __uint_as_float(wd[j][k][0]);
            x1 = __uint_as_float(wd[j][k][EW - 1]);
          } else if constexpr (DT == DT_BF16) {
            x0 = __uint_as_float(wd[j][k][0] << 16);
            x1 = __uint_as_float(wd[j][k][0] & 0xffff0000u);
          } else {
            x0 = f16_value(wd[j][k][0] & 0xffffu);
            x1 = f16_value(wd[j][k][0] >> 16);
          }
          float y0 = x0, y1 = x1;
          if (a.rope) {
            y0 = __builtin_fmaf(x0, c[k], -x1 * sn[k]);
            y1 = __builtin_fmaf(x0, sn[k], x1 * c[k]);
          }
          b0 += fabsf(y0);
          b1 += fabsf(y1);
        }
        s0[k] += (double)b0;
        s1[k] += (double)b1;
      }
    }
  }
  double* pb = a.part + w * D;
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int i = lane + 64 * k;
    pb[2 * i] = s0[k];
    pb[2 * i + 1] = s1[k];
  }
}

// stats[c] = (sum over waves of the per-wave sums) / (vectors counted), in a fixed order
// (deterministic) and in two steps that read the partials along their rows: channel_stats_runs
// adds runs of kStatRun consecutive waves (block j: waves j kStatRun ..; thread = channel) and
// writes each run's sums over the run's first row, which no other block reads; then
// channel_stats_final adds the runs in order and divides (one thread per channel).  One block
// per channel reading a column at a 1-KiB stride took 19 us at 8192 waves.
constexpr int kStatRun = 64;
template <int D>
__global__ void __launch_bounds__(256) channel_stats_runs(const CalibArgs a) {
  const int64_t w0 = (int64_t)blockIdx.x * kStatRun;
  const int c = threadIdx.x;
  if (c >= D) return;
  const int64_t w1 = min(w0 + (int64_t)kStatRun, a.n_waves);
  double s = 0.0;
#pragma unroll 8
  for (int64_t w = w0; w < w1; ++w) s += a.part[w * D + c];
  a.part[w0 * D + c] = s;  // thread c alone reads and writes column c of this run
}
template <int D>
__global__ void __launch_bounds__(256) channel_stats_final(const CalibArgs a) {
  const int c = threadIdx.x;
  if (c >= D) return;
  double s = 0.0;
#pragma unroll 8
  for (int64_t w0 = 0; w0 < a.n_waves; w0 += kStatRun) s += a.part[w0 * D + c];
  int64_t sink = (int64_t)a.n_sink - a.pos_offset;
  sink = sink < 0 ? 0 : (sink > a.tokens ? a.tokens : sink);
  const double n = (double)(a.rows * a.heads * (a.tokens - sink));
  a.stats[c] = n > 0.0 ? s / n : 0.0;
}

// Token norms: one wave per (row, token); the token's heads are read in 16-byte pieces, the
// squares summed in float64 (exact for 16-bit inputs: each square has at most 22 significant
// bits, and float32 squares at most 48), then reduced across the wave.
template <int DT, int D>
__global__ void __launch_bounds__(256) token_norm_kernel(const CalibArgs a) {
  constexpr int ES = (DT == DT_F32) ? 4 : 2;
  constexpr int CPV = D * ES / 16;  // 16-byte pieces per vector
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= a.rows * a.tokens) return;  // wave-uniform
  const int64_t r = w / a.tokens, t = w % a.tokens;
  const char* base = reinterpret_cast<const char*>(a.x) + (r * a.sr + t * a.st) * ES;
  // streamed loads (each line is read once, whole: measured 6 % faster than temporal ones);
  // the token's head span is below 2^31 bytes (checked on the host)
  const buf_t tb = make_buf(base, ((a.heads - 1) * a.sh + D) * ES);
  double acc = 0.0;
  for (int64_t k = lane; k < a.heads * CPV; k += 64) {
    const int64_t h = k / CPV, cc = k % CPV;
    const u32x4_t q = __builtin_amdgcn_raw_buffer_load_b128(tb, (uint32_t)(h * a.sh * ES + 16 * cc), 0, kNT | kSC1);
    const uint32_t ws[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (DT == DT_F32) {
        const double x = (double)__uint_as_float(ws[e]);
        acc = __builtin_fma(x, x, acc);
      } else {
        const double x0 = (double)(DT == DT_BF16 ? __uint_as_float(ws[e] << 16) : f16_value(ws[e] & 0xffffu));
        const double x1 = (double)(DT == DT_BF16 ? __uint_as_float(ws[e] & 0xffff0000u) : f16_value(ws[e] >> 16));
        acc = __builtin_fma(x0, x0, acc);
        acc = __builtin_fma(x1, x1, acc);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) a.norms[w] = __builtin_sqrt(acc);
}

// Per row: the lower median of the T token norms by an exact radix select on their bit
// patterns (non-negative doubles order as unsigned integers), eight 8-bit digits from the top;
// then the flags (norm > lambda * median), their count and one past the last flagged token.
// One block of kSelectThreads per row; each digit's bin is found by one wave (4 bins per lane,
// an inclusive scan of the lane sums).  Rows of up to kSelectHeld * kSelectThreads tokens are
// read once into registers; longer rows are read again for every digit.
constexpr int kSelectThreads = 1024;
constexpr int kSelectHeld = 32;
__global__ void __launch_bounds__(kSelectThreads) sink_select_kernel(const CalibArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ int64_t s_k;
  __shared__ int s_b;
  __shared__ int s_count, s_last;
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t T = a.tokens;
  const double* nr = a.norms + r * T;
  if (T == 0) {
    if (tid == 0) {
      a.counts[r] = 0;
      a.prefix[r] = 0;
      a.medians[r] = 0.0;
    }
    return;  // block-uniform
  }
  const bool held = T <= (int64_t)kSelectHeld * kSelectThreads;  // block-uniform
  uint64_t hv[kSelectHeld];
  if (held) {
#pragma unroll
    for (int i = 0; i < kSelectHeld; ++i) {
      const int64_t t = tid + (int64_t)i * kSelectThreads;
      hv[i] = t < T ? (uint64_t)__double_as_longlong(nr[t]) : 0u;
    }
  }
  uint64_t prefix = 0, mask = 0;
  int64_t k = (T - 1) / 2;  // rank of the lower median among the values that match the prefix
  for (int d = 7; d >= 0; --d) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    // a thread's values fall into one bin over long runs in the top digits (the exponent), so it
    // counts a run in a register and adds it with one atomic when the bin changes
    uint32_t run_bin = 0u, run_n = 0u;
    auto count = [&](uint64_t v) __attribute__((always_inline)) {
      if ((v & mask) == prefix) {
        const uint32_t b = (uint32_t)(v >> (8 * d)) & 255u;
        if (b != run_bin) {
          if (run_n) atomicAdd(&hist[run_bin], run_n);
          run_bin = b;
          run_n = 0u;
        }
        ++run_n;
      }
    };
    if (held) {
#pragma unroll
      for (int i = 0; i < kSelectHeld; ++i)
        if (tid + (int64_t)i * kSelectThreads < T) count(hv[i]);
    } else {
      for (int64_t t = tid; t < T; t += kSelectThreads) count((uint64_t)__double_as_longlong(nr[t]));
    }
    if (run_n) atomicAdd(&hist[run_bin], run_n);
    __syncthreads();
    if (tid < 64) {
      // lane L: bins 4L .. 4L + 3; the digit is the bin where the running count passes k
      // (exactly one lane holds it: the matching values number more than k)
      uint32_t hb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) hb[e] = hist[4 * tid + e];
      // counts stay below T < 2^31 (tokens * heads < 2^31 on the host)
      const int own = (int)(hb[0] + hb[1] + hb[2] + hb[3]);
      int incl = own;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int up = __shfl_up(incl, o);
        if (tid >= o) incl += up;
      }
      int64_t below = incl - own;
      if (below <= k && k < incl) {
        int e = 0;
        for (; e < 3; ++e) {
          if (below + (int64_t)hb[e] > k) break;
          below += hb[e];
        }
        s_k = k - below;
        s_b = 4 * tid + e;
      }
    }
    __syncthreads();
    k = s_k;
    prefix |= (uint64_t)s_b << (8 * d);
    mask |= (uint64_t)255u << (8 * d);
    __syncthreads();  // every thread has read s_k and s_b before the next digit's histogram
  }
  const double med = __longlong_as_double((long long)prefix);
  if (tid == 0) {
    s_count = 0;
    s_last = -1;
  }
  __syncthreads();
  const double thr = a.lambda * med;
  int cnt = 0, last = -1;
  for (int64_t t = tid; t < T; t += kSelectThreads) {
    const bool f = nr[t] > thr;
    a.flags[r * T + t] = f ? 1 : 0;
    cnt += f ? 1 : 0;
    last = f ? (int)t : last;
  }
  atomicAdd(&s_count, cnt);
  atomicMax(&s_last, last);
  __syncthreads();
  if (tid == 0) {
    a.counts[r] = s_count;
    a.prefix[r] = s_last + 1;
    a.medians[r] = med;
  }
}

// Rotated moments for the dynamic codebook: the codec's front end (RoPE, norm separation,
// permutation, rotation) on each vector, then per rotated channel the sum of z^2.  One wave per
// (row, run of tokens), one vector at a time: lane i holds channels i + 64 k (k < D/64), so the
// channel bits 0..5 are lane bits (shuffles) and the rest register bits.
template <int DT, int D>
__global__ void __launch_bounds__(256) rotated_moments_kernel(const CalibArgs a) {
  constexpr int K = D / 64;
  constexpr int ES = (DT == DT_F32) ? 4 : 2;
  __shared__ float s_mat[(D / 4) * 16];
  __shared__ float s_u[4][D];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (a.rot == ROT_SO4)
    for (int b = threadIdx.x; b < D / 4; b += blockDim.x) build_so4(&a.quat[8 * b], &s_mat[16 * b]);
  __syncthreads();
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= a.n_waves) return;  // wave-uniform; no barrier follows
  const int64_t nchunk = (a.tokens + a.tpw - 1) / a.tpw;
  const int64_t r = w / nchunk, t0 = (w % nchunk) * a.tpw;
  const int64_t t1 = min(t0 + (int64_t)a.tpw, a.tokens);
  double theta[K], acc[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    theta[k] = exp2(-(2.0 * (double)((lane + 64 * k) >> 1) / (double)D) * a.rope_log2_base);
    acc[k] = 0.0;
  }
  const float norm_c = (float)(1.0 / __builtin_sqrt((double)D));
  const char* base = reinterpret_cast<const char*>(a.x);
  for (int64_t t = t0; t < t1; ++t) {
    const int64_t pos = a.pos_offset + t;
    if (pos < a.n_sink) continue;  // wave-uniform
    float c[K], sn[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      c[k] = 1.0f;
      sn[k] = 0.0f;
      if (a.rope) rope_cos_sin(pos, theta[k], &c[k], &sn[k]);
    }
    for (int64_t h = 0; h < a.heads; ++h) {
      const char* vp = base + (r * a.sr + t * a.st + h * a.sh) * ES;
      float u[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int ch = lane + 64 * k;
        if constexpr (DT == DT_F32) u[k] = reinterpret_cast<const float*>(vp)[ch];
        else if constexpr (DT == DT_BF16) u[k] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(vp)[ch] << 16);
        else u[k] = f16_value(reinterpret_cast<const uint16_t*>(vp)[ch]);
      }
      if (a.rope) {  // pair (2i, 2i + 1) = lanes (2m, 2m + 1) of the same register
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float p = __shfl_xor(u[k], 1);
          u[k] = (lane & 1) ? __builtin_fmaf(p, sn[k], u[k] * c[k]) : __builtin_fmaf(u[k], c[k], -p * sn[k]);
        }
      }
      // norm separation: u / (rho + 1e-6)
      float ss = 0.0f;
#pragma unroll
      for (int k = 0; k < K; ++k) ss = __builtin_fmaf(u[k], u[k], ss);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
      const float inv = 1.0f / (__builtin_sqrtf(ss) + 1e-6f);
#pragma unroll
      for (int k = 0; k < K; ++k) u[k] *= inv;
      if (a.use_perm) {  // u'[c] = u[perm[c]]
        float v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const int src = a.perm[lane + 64 * k];
          float val = 0.0f;
#pragma unroll
          for (int kk = 0; kk < K; ++kk) {
            const float x = __shfl(u[kk], src & 63);
            val = (src >> 6) == kk ? x : val;
          }
          v[k] = val;
        }
#pragma unroll
        for (int k = 0; k < K; ++k) u[k] = v[k];
      }
      float z[K];
      if (a.rot == ROT_FWHT) {
        // bits 6.. in the lane (registers), bits 0..5 across lanes; then 1/sqrt(D)
#pragma unroll
        for (int hb = 1; hb < K; hb <<= 1)
#pragma unroll
          for (int k = 0; k < K; ++k)
            if (!(k & hb)) {
              const float x = u[k], y = u[k + hb];
              u[k] = x + y;
              u[k + hb] = x - y;
            }
#pragma unroll
        for (int bit = 1; bit < 64; bit <<= 1)
#pragma unroll
          for (int k = 0; k < K; ++k) {
            const float p = __shfl_xor(u[k], bit);
            u[k] = (lane & bit) ? p - u[k] : u[k] + p;
          }
#pragma unroll
        for (int k = 0; k < K; ++k) z[k] = u[k] * norm_c;
      } else if (a.rot == ROT_SO4) {  // block b = channels 4b .. 4b + 3 = lanes 4m .. 4m + 3
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const int ch = lane + 64 * k, b = ch >> 2, row = ch & 3;
          float acc4 = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc4 = __builtin_fmaf(s_mat[16 * b + 4 * row + i], __shfl(u[k], (lane & ~3) + i), acc4);
          z[k] = acc4;
        }
      } else if (a.rot == ROT_DENSE) {  // z_i = sum_j M[i][j] u_j, u staged in LDS
        float* su = s_u[wave];
#pragma unroll
        for (int k = 0; k < K; ++k) su[lane + 64 * k] = u[k];
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float* row = a.rot_matrix + (int64_t)(lane + 64 * k) * D;
          float acc1 = 0.0f;
          for (int j = 0; j < D; ++j) acc1 = __builtin_fmaf(row[j], su[j], acc1);
          z[k] = acc1;
        }
        wave_lds_sync();
      } else {
#pragma unroll
        for (int k = 0; k < K; ++k) z[k] = u[k];
      }
#pragma unroll
      for (int k = 0; k < K; ++k) acc[k] += (double)z[k] * (double)z[k];
    }
  }
  double* pb = a.part + w * D;
#pragma unroll
  for (int k = 0; k < K; ++k) pb[lane + 64 * k] = acc[k];
}

// ---------------------------------------------------------------------------
// Attention entropy (dynamic bit width): per (row, query head) the entropy of the softmax over
// the row's slots, scored in the rotated domain as the attention does (q . k = (M P q) . y).
// ---------------------------------------------------------------------------
// rotated queries: one wave per (row, query head); lane i holds channels i + 64 k
template <int D>
__global__ void __launch_bounds__(256) entropy_rotate_q(const EntropyArgs a) {
  constexpr int K = D / 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= a.rows * a.q_heads) return;  // wave-uniform; no barrier in this kernel
  const float* q = a.q + w * D;
  float u[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int c = lane + 64 * k;
    u[k] = q[a.use_perm ? a.perm[c] : c];  // (P q)[c] = q[perm[c]]
  }
#pragma unroll
  for (int hb = 1; hb < K; hb <<= 1)
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (!(k & hb)) {
        const float x = u[k], y = u[k + hb];
        u[k] = x + y;
        u[k + hb] = x - y;
      }
#pragma unroll
  for (int bit = 1; bit < 64; bit <<= 1)
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const float p = __shfl_xor(u[k], bit);
      u[k] = (lane & bit) ? p - u[k] : u[k] + p;
    }
  const float nc = (float)(1.0 / __builtin_sqrt((double)D));
#pragma unroll
  for (int k = 0; k < K; ++k) a.qrot[w * D + lane + 64 * k] = u[k] * nc;
}

// online (max, L = sum e^(s - max), S = sum e^(s - max) (s - max)) with one more score
__device__ __forceinline__ void ent_push(float& M, float& L, float& S, float s) {
  if (s > M) {
    if (M == -INFINITY) {  // the first score: nothing to rescale (and -inf * 0 would be NaN)
      L = 0.0f;
      S = 0.0f;
    } else {
      const float f = __expf(M - s);
      S = f * (S + (M - s) * L);
      L = f * L;
    }
    M = s;
  }
  const float p = __expf(s - M);
  L += p;
  S = __builtin_fmaf(p, s - M, S);
}
// (M, L, S) merged with another triple
__device__ __forceinline__ void ent_merge(float& M, float& L, float& S, float M2, float L2, float S2) {
  if (M2 == -INFINITY) return;
  if (M == -INFINITY) {
    M = M2;
    L = L2;
    S = S2;
    return;
  }
  const float Mn = fmaxf(M, M2);
  const float f1 = __expf(M - Mn), f2 = __expf(M2 - Mn);
  S = f1 * (S + (M - Mn) * L) + f2 * (S2 + (M2 - Mn) * L2);
  L = f1 * L + f2 * L2;
  M = Mn;
}

// Partial pass: one wave per (row, KV head, chunk of slots); each lane scores its own slots
// (t = t_begin + lane + 64 i) against the QG rotated queries held in LDS.
template <int D, int BITS, int QG>
__global__ void __launch_bounds__(256) entropy_partial(const EntropyArgs a) {
  constexpr int CB = D * BITS / 8;  // code bytes per vector
  __shared__ float s_q[4][QG * D];
  __shared__ float s_qs[4][QG * (D / 32)];  // per query head and group: the sum of its channels
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= a.rows * a.heads * a.n_chunks) return;  // wave-uniform; no block barrier follows
  const int64_t c = w % a.n_chunks, rh = w / a.n_chunks, h = rh % a.heads, r = rh / a.heads;
  int64_t len = a.tokens;
  if (a.lengths) {
    const int64_t n = a.lengths[r];
    len = n < 0 ? 0 : (n > a.tokens ? a.tokens : n);
  }
  const int64_t t_begin = max(c * (int64_t)a.chunk, (int64_t)a.n_sink);
  const int64_t t_end = min((c + 1) * (int64_t)a.chunk, len);
  float* sq = s_q[wave];
  const float* src = a.qrot + (r * a.q_heads + h * QG) * D;
  for (int i = lane; i < QG * D; i += 64) sq[i] = src[i];
  wave_lds_sync();
  const int G = 1 << a.group_log2, ng = D >> a.group_log2;
  // the group sums of the queries, once per wave (in channel order, as a slot's pass would)
  for (int i = lane; i < QG * ng; i += 64) {
    const int m = i / ng, g0 = (i % ng) * G;
    float acc = 0.0f;
    for (int j = 0; j < G; ++j) acc += sq[m * D + g0 + j];
    s_qs[wave][i] = acc;
  }
  wave_lds_sync();
  float M[QG], L[QG], S[QG];
#pragma unroll
  for (int m = 0; m < QG; ++m) {
    M[m] = -INFINITY;
    L[m] = 0.0f;
    S[m] = 0.0f;
  }
  for (int64_t t = t_begin + lane; t < t_end; t += 64) {
    const int64_t vec = (r * a.tokens + t) * a.heads + h;
    const uint32_t* cw = reinterpret_cast<const uint32_t*>(a.k_codes + vec * CB);
    float dot[QG], sc[QG];
#pragma unroll
    for (int m = 0; m < QG; ++m) {
      sc[m] = 0.0f;
      dot[m] = 0.0f;
    }
    // blocks of 32 channels (BITS code words each; groups are whole blocks)
#pragma unroll 1
    for (int blk = 0; blk < D / 32; ++blk) {
      uint32_t wd[BITS];
#pragma unroll
      for (int k = 0; k < BITS; ++k) wd[k] = cw[BITS * blk + k];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int bit = BITS * i, wi = bit >> 5, sh = bit & 31;
        uint32_t code = wd[wi] >> sh;
        if (BITS == 3 && sh > 29) code |= wd[wi + 1] << (32 - sh);
        const float cf = (float)(code & ((1u << BITS) - 1u));
#pragma unroll
        for (int m = 0; m < QG; ++m) {
          dot[m] = __builtin_fmaf(sq[m * D + 32 * blk + i], cf, dot[m]);
        }
      }
      if ((((blk + 1) << 5) & (G - 1)) == 0) {  // the end of a group: q . (zero + code * scale)
        const int g = (32 * blk) >> a.group_log2;
        const float gs = f16_value(a.k_scale[vec * ng + g]), gz = f16_value(a.k_zero[vec * ng + g]);
#pragma unroll
        for (int m = 0; m < QG; ++m) {
          sc[m] = __builtin_fmaf(gs, dot[m], __builtin_fmaf(gz, s_qs[wave][m * ng + g], sc[m]));
          dot[m] = 0.0f;
        }
      }
    }
#pragma unroll
    for (int m = 0; m < QG; ++m) ent_push(M[m], L[m], S[m], sc[m] * a.scale);
  }
  // merge the wave's lanes, write the chunk's partial for each query head
#pragma unroll
  for (int m = 0; m < QG; ++m) {
    float Mm = M[m], Lm = L[m], Sm = S[m];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float M2 = __shfl_xor(Mm, o), L2 = __shfl_xor(Lm, o), S2 = __shfl_xor(Sm, o);
      ent_merge(Mm, Lm, Sm, M2, L2, S2);
    }
    if (lane == 0) {
      float* pb = a.part + ((r * a.q_heads + h * QG + m) * a.n_chunks + c) * 4;
      pb[0] = Mm;
      pb[1] = Lm;
      pb[2] = Sm;
    }
  }
}

// Merge the chunks and the fp16 sink slots (raw query against unrotated keys); H = ln L - S / L.
template <int D>
__global__ void __launch_bounds__(256) entropy_combine(const EntropyArgs a) {
  constexpr int K = D / 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= a.rows * a.q_heads) return;  // wave-uniform; no barrier in this kernel
  const int64_t r = w / a.q_heads, m = w % a.q_heads;
  const int64_t h = m / (a.q_heads / a.heads);
  int64_t len = a.tokens;
  if (a.lengths) {
    const int64_t n = a.lengths[r];
    len = n < 0 ? 0 : (n > a.tokens ? a.tokens : n);
  }
  // lane i merges chunks i, i + 64, ...; then the lanes merge by a butterfly (the merge is
  // symmetric in its two operands, so every lane ends with the same values)
  float M = -INFINITY, L = 0.0f, S = 0.0f;
  for (int c = lane; c < a.n_chunks; c += 64) {
    const float* pb = a.part + (w * a.n_chunks + c) * 4;
    ent_merge(M, L, S, pb[0], pb[1], pb[2]);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float M2 = __shfl_xor(M, o), L2 = __shfl_xor(L, o), S2 = __shfl_xor(S, o);
    ent_merge(M, L, S, M2, L2, S2);
  }
  const int nsk = (int)min((int64_t)a.n_sink, len);
  const float* qr = a.q + w * D;
  float qv[K];
#pragma unroll
  for (int k = 0; k < K; ++k) qv[k] = qr[lane + 64 * k];
  for (int t = 0; t < nsk; ++t) {
    const uint16_t* kk = a.k_sink + ((r * a.n_sink + t) * a.heads + h) * D;
    float d = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) d = __builtin_fmaf(qv[k], f16_value(kk[lane + 64 * k]), d);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) d += __shfl_xor(d, o);
    ent_push(M, L, S, d * a.scale);
  }
  if (lane == 0) a.entropy[w] = L > 0.0f ? __logf(L) - S / L : 0.0f;
}

template <int D, int BITS, int QG>
int launch_entropy_t(const EntropyArgs& a, hipStream_t s) {
  const int64_t nq = a.rows * a.q_heads, np = a.rows * a.heads * a.n_chunks;
  if (nq == 0) return 0;
  hipLaunchKernelGGL((entropy_rotate_q<D>), dim3((unsigned)((nq + 3) / 4)), dim3(256), 0, s, a);
  if (hipError_t e = hipGetLastError()) return (int)e;
  hipLaunchKernelGGL((entropy_partial<D, BITS, QG>), dim3((unsigned)((np + 3) / 4)), dim3(256), 0, s, a);
  if (hipError_t e = hipGetLastError()) return (int)e;
  hipLaunchKernelGGL((entropy_combine<D>), dim3((unsigned)((nq + 3) / 4)), dim3(256), 0, s, a);
  return (int)hipGetLastError();
}
template <int D, int BITS>
int pick_entropy_qg(const EntropyArgs& a, hipStream_t s) {
  switch (a.q_heads / a.heads) {
    case 1: return launch_entropy_t<D, BITS, 1>(a, s);
    case 2: return launch_entropy_t<D, BITS, 2>(a, s);
    case 4: return launch_entropy_t<D, BITS, 4>(a, s);
    default: return launch_entropy_t<D, BITS, 8>(a, s);
  }
}

template <int DT, int D>
int launch_moments_t(const CalibArgs& a, hipStream_t s) {
  if (a.n_waves > 0) {
    hipLaunchKernelGGL((rotated_moments_kernel<DT, D>), dim3((unsigned)((a.n_waves + 3) / 4)), dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError()) return (int)e;
    hipLaunchKernelGGL((channel_stats_runs<D>), dim3((unsigned)((a.n_waves + kStatRun - 1) / kStatRun)), dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError()) return (int)e;
  }
  hipLaunchKernelGGL((channel_stats_final<D>), dim3(1), dim3(256), 0, s, a);
  return (int)hipGetLastError();
}

template <int DT, int D>
int launch_stats_t(const CalibArgs& a, hipStream_t s) {
  if (a.n_waves > 0) {
    hipLaunchKernelGGL((channel_stats_kernel<DT, D>), dim3((unsigned)((a.n_waves + 3) / 4)), dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError()) return (int)e;
    hipLaunchKernelGGL((channel_stats_runs<D>), dim3((unsigned)((a.n_waves + kStatRun - 1) / kStatRun)), dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError()) return (int)e;
  }
  // (an empty slice still gets its statistics written: all zero)
  hipLaunchKernelGGL((channel_stats_final<D>), dim3(1), dim3(256), 0, s, a);
  return (int)hipGetLastError();
}
template <int DT, int D>
int launch_sinks_t(const CalibArgs& a, hipStream_t s) {
  if (a.rows == 0) return 0;
  const int64_t nw = a.rows * a.tokens;
  if (nw > 0) {
    hipLaunchKernelGGL((token_norm_kernel<DT, D>), dim3((unsigned)((nw + 3) / 4)), dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError()) return (int)e;
  }
  hipLaunchKernelGGL(sink_select_kernel, dim3((unsigned)a.rows), dim3(kSelectThreads), 0, s, a);
  return (int)hipGetLastError();
}
}  // namespace

int launch_channel_stats(const CalibArgs& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool d128 = a.head_dim == 128;
  switch (a.dtype) {
    case DT_F16: return d128 ? launch_stats_t<DT_F16, 128>(a, s) : launch_stats_t<DT_F16, 256>(a, s);
    case DT_BF16: return d128 ? launch_stats_t<DT_BF16, 128>(a, s) : launch_stats_t<DT_BF16, 256>(a, s);
    default: return d128 ? launch_stats_t<DT_F32, 128>(a, s) : launch_stats_t<DT_F32, 256>(a, s);
  }
}
int launch_entropy(const EntropyArgs& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a.head_dim == 128) {
    if (a.bits == 2) return pick_entropy_qg<128, 2>(a, s);
    if (a.bits == 3) return pick_entropy_qg<128, 3>(a, s);
    return pick_entropy_qg<128, 4>(a, s);
  }
  if (a.bits == 2) return pick_entropy_qg<256, 2>(a, s);
  if (a.bits == 3) return pick_entropy_qg<256, 3>(a, s);
  return pick_entropy_qg<256, 4>(a, s);
}
int launch_rotated_moments(const CalibArgs& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool d128 = a.head_dim == 128;
  switch (a.dtype) {
    case DT_F16: return d128 ? launch_moments_t<DT_F16, 128>(a, s) : launch_moments_t<DT_F16, 256>(a, s);
    case DT_BF16: return d128 ? launch_moments_t<DT_BF16, 128>(a, s) : launch_moments_t<DT_BF16, 256>(a, s);
    default: return d128 ? launch_moments_t<DT_F32, 128>(a, s) : launch_moments_t<DT_F32, 256>(a, s);
  }
}
int launch_detect_sinks(const CalibArgs& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool d128 = a.head_dim == 128;
  switch (a.dtype) {
    case DT_F16: return d128 ? launch_sinks_t<DT_F16, 128>(a, s) : launch_sinks_t<DT_F16, 256>(a, s);
    case DT_BF16: return d128 ? launch_sinks_t<DT_BF16, 128>(a, s) : launch_sinks_t<DT_BF16, 256>(a, s);
    default: return d128 ? launch_sinks_t<DT_F32, 128>(a, s) : launch_sinks_t<DT_F32, 256>(a, s);
  }
}
#endif

}  // namespace kvq
