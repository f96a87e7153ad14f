// Host side of the kvq C ABI: argument checking, plane sizes, kernel-argument
// marshalling and dispatch.  Every check runs before anything is enqueued, so
// an error return means no work was done.  No HIP call is made on an error path.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/kvq.h"
#include "kvq_internal.h"

namespace {

thread_local std::string g_last_error;

kvq_status fail(kvq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kvq_status ok() {
  g_last_error.clear();
  return KVQ_OK;
}

int elem_size(int dtype) { return dtype == KVQ_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int ilog2(int64_t v) {
  int r = 0;
  while ((int64_t(1) << r) < v) ++r;
  return r;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

struct Derived {
  int64_t n_vec = 0;        // R*T*H
  int64_t sr = 0, st = 0, sh = 0;
  int64_t code_bytes = 0;   // per vector
  int64_t ngroups = 0;      // per vector (min-max)
  int64_t extra_bytes = 0;  // per vector (dynamic codebook)
};

kvq_status check_config(const kvq_config* cfg, Derived* dv) {
  if (!cfg) return fail(KVQ_ERR_NULL, "cfg is NULL");
  if (cfg->abi_version != KVQ_ABI_VERSION)
    return fail(KVQ_ERR_ABI, "abi_version %d, library is %d", cfg->abi_version, KVQ_ABI_VERSION);
  if (cfg->dtype < KVQ_F16 || cfg->dtype > KVQ_F32) return fail(KVQ_ERR_ROT, "unknown dtype %d", cfg->dtype);
  if (cfg->rot < KVQ_ROT_NONE || cfg->rot > KVQ_ROT_ROTOR) return fail(KVQ_ERR_ROT, "unknown rotation %d", cfg->rot);
  if (cfg->quant < KVQ_Q_MINMAX || cfg->quant > KVQ_Q_LLOYD)
    return fail(KVQ_ERR_ROT, "unknown quantizer %d", cfg->quant);
  if (cfg->rows < 0 || cfg->tokens < 0 || cfg->heads < 0 || cfg->head_dim < 0)
    return fail(KVQ_ERR_SHAPE, "negative size");
  const int64_t d = cfg->head_dim;
  if (d != 128 && d != 256) return fail(KVQ_ERR_UNSUPPORTED, "head_dim %lld (supported: 128, 256)", (long long)d);
  if (cfg->bits < 2 || cfg->bits > 4) return fail(KVQ_ERR_BITS, "bits %d (supported: 2, 3, 4)", cfg->bits);
  if (cfg->quant == KVQ_Q_MINMAX) {
    const int g = cfg->group_size;
    if (!(g == 32 || g == 64 || g == 128 || g == 256) || g > d)
      return fail(KVQ_ERR_GROUP, "group_size %d (32, 64, 128 or 256, at most head_dim)", g);
  }
  int64_t th = 0, rth = 0, n = 0;
  if (!mul_ok(cfg->tokens, cfg->heads, &th) || !mul_ok(cfg->rows, th, &rth) || !mul_ok(rth, d, &n) ||
      n > (int64_t(1) << 50))
    return fail(KVQ_ERR_SHAPE, "tensor too large");
  if (th >= (int64_t(1) << 31)) return fail(KVQ_ERR_SHAPE, "tokens*heads must be below 2^31");
  if (cfg->heads > 32768) return fail(KVQ_ERR_SHAPE, "heads %lld (at most 32768)", (long long)cfg->heads);
  if (cfg->rope != 0 && cfg->rope != 1) return fail(KVQ_ERR_PARAM, "rope must be 0 or 1");
  if (cfg->rope && !(isfinite(cfg->rope_base) && cfg->rope_base > 1.0))
    return fail(KVQ_ERR_PARAM, "rope_base must be finite and > 1");
  // (tokens >= 0 here, so the right-hand side cannot overflow; pos_offset + tokens could)
  if (cfg->pos_offset < 0 || cfg->pos_offset > (int64_t(1) << 31) - cfg->tokens)
    return fail(KVQ_ERR_PARAM, "positions must lie in [0, 2^31]");
  if (cfg->n_sink < 0) return fail(KVQ_ERR_PARAM, "n_sink must be >= 0");

  // strides
  const int es = elem_size(cfg->dtype);
  if (cfg->stride_r == 0 && cfg->stride_t == 0 && cfg->stride_h == 0) {
    dv->sh = d;
    dv->st = cfg->heads * d;
    dv->sr = cfg->tokens * cfg->heads * d;
  } else {
    if (cfg->stride_r < 0 || cfg->stride_t < 0 || cfg->stride_h < 0)
      return fail(KVQ_ERR_SHAPE, "negative stride");
    const int64_t unit = 16 / es;
    if (cfg->stride_r % unit || cfg->stride_t % unit || cfg->stride_h % unit)
      return fail(KVQ_ERR_ALIGN, "strides must be multiples of %lld elements (16 bytes)", (long long)unit);
    int64_t tmp;
    if (!mul_ok(cfg->stride_r, std::max<int64_t>(cfg->rows, 1), &tmp) ||
        !mul_ok(cfg->stride_t, std::max<int64_t>(cfg->tokens, 1), &tmp) ||
        !mul_ok(cfg->stride_h, std::max<int64_t>(cfg->heads, 1), &tmp))
      return fail(KVQ_ERR_SHAPE, "strided extent overflows");
    dv->sr = cfg->stride_r;
    dv->st = cfg->stride_t;
    dv->sh = cfg->stride_h;
  }
  // the kernels address a wave's 16 (or 8) vectors of one row from a common base with
  // 32-bit lane offsets: 16 token strides plus a head span must stay below 2^31 bytes
  {
    const double span = (16.0 * (double)dv->st + (double)std::max<int64_t>(cfg->heads - 1, 0) * (double)dv->sh +
                         (double)d) * es;
    if (span >= 2147483648.0) return fail(KVQ_ERR_SHAPE, "token/head strides too large (16 token strides must span < 2 GiB)");
  }

  // parameters
  if (cfg->perm) {
    bool seen[kvq::kMaxHeadDim] = {false};
    for (int64_t i = 0; i < d; ++i) {
      const uint16_t p = cfg->perm[i];
      if (p >= d || seen[p]) return fail(KVQ_ERR_PARAM, "perm is not a permutation of 0..%lld", (long long)(d - 1));
      seen[p] = true;
    }
  }
  if (cfg->rot == KVQ_ROT_SO4) {
    if (!cfg->quat) return fail(KVQ_ERR_NULL, "quat is required for the SO(4) rotation");
    for (int64_t b = 0; b < d / 4; ++b)
      for (int side = 0; side < 2; ++side) {
        const float* q = cfg->quat + 8 * b + 4 * side;
        double s = 0.0;
        for (int i = 0; i < 4; ++i) {
          if (!isfinite(q[i])) return fail(KVQ_ERR_PARAM, "quaternion %lld is not finite", (long long)b);
          s += (double)q[i] * q[i];
        }
        if (fabs(sqrt(s) - 1.0) > 1e-4) return fail(KVQ_ERR_PARAM, "quaternion %lld is not unit", (long long)b);
      }
  }
  if (cfg->rot == KVQ_ROT_ROTOR) {
    if (!cfg->rotor_quat) return fail(KVQ_ERR_NULL, "rotor_quat is required for the rotor rotation");
    for (int64_t b = 0; b < d / 3; ++b) {
      const float* q = cfg->rotor_quat + 4 * b;
      double s = 0.0;
      for (int i = 0; i < 4; ++i) {
        if (!isfinite(q[i])) return fail(KVQ_ERR_PARAM, "rotor %lld is not finite", (long long)b);
        s += (double)q[i] * q[i];
      }
      if (fabs(sqrt(s) - 1.0) > 1e-4) return fail(KVQ_ERR_PARAM, "rotor %lld is not unit", (long long)b);
    }
    if (!isfinite(cfg->rotor_tail)) return fail(KVQ_ERR_PARAM, "rotor_tail must be finite");
  }
  if (cfg->quant == KVQ_Q_LLOYD) {
    if (!cfg->codebook) return fail(KVQ_ERR_NULL, "codebook is required for Lloyd-Max");
    const int n_levels = 1 << cfg->bits;
    for (int i = 0; i < n_levels; ++i) {
      if (!isfinite(cfg->codebook[i])) return fail(KVQ_ERR_PARAM, "codebook entry %d not finite", i);
      if (i > 0 && !(cfg->codebook[i] > cfg->codebook[i - 1]))
        return fail(KVQ_ERR_PARAM, "codebook not strictly ascending at %d", i);
    }
  }
  // dynamic codebook
  const bool any_dyn = cfg->chan_scale || cfg->chan_wide || cfg->codebook_wide;
  if (any_dyn) {
    if (!cfg->chan_scale || !cfg->chan_wide || !cfg->codebook_wide)
      return fail(KVQ_ERR_NULL, "the dynamic codebook needs chan_scale, chan_wide and codebook_wide");
    if (cfg->quant != KVQ_Q_LLOYD) return fail(KVQ_ERR_PARAM, "the dynamic codebook is a Lloyd-Max codebook");
    int n_wide = 0;
    for (int64_t j = 0; j < d; ++j) {
      if (!(isfinite(cfg->chan_scale[j]) && cfg->chan_scale[j] > 0.0f))
        return fail(KVQ_ERR_PARAM, "chan_scale[%lld] must be finite and > 0", (long long)j);
      if (cfg->chan_wide[j] > 1) return fail(KVQ_ERR_PARAM, "chan_wide[%lld] must be 0 or 1", (long long)j);
      n_wide += cfg->chan_wide[j];
    }
    if (n_wide != d / 16) return fail(KVQ_ERR_PARAM, "chan_wide has %d ones, head_dim/16 = %lld needed", n_wide,
                                      (long long)(d / 16));
    const int n_levels = 2 << cfg->bits;
    for (int i = 0; i < n_levels; ++i) {
      if (!isfinite(cfg->codebook_wide[i])) return fail(KVQ_ERR_PARAM, "codebook_wide entry %d not finite", i);
      if (i > 0 && !(cfg->codebook_wide[i] > cfg->codebook_wide[i - 1]))
        return fail(KVQ_ERR_PARAM, "codebook_wide not strictly ascending at %d", i);
    }
  }
  if (cfg->rot == KVQ_ROT_DENSE) {
    if (!cfg->rot_matrix) return fail(KVQ_ERR_NULL, "rot_matrix is required for the dense rotation");
    if (!aligned16(cfg->rot_matrix)) return fail(KVQ_ERR_ALIGN, "rot_matrix not 16-byte aligned");
  }
  dv->n_vec = rth;
  dv->code_bytes = d * cfg->bits / 8;
  dv->ngroups = cfg->quant == KVQ_Q_MINMAX ? d / cfg->group_size : 0;
  dv->extra_bytes = any_dyn ? d / 128 : 0;
  return KVQ_OK;
}

void plane_sizes(const kvq_config* cfg, const Derived& dv, size_t* codes, size_t* scale, size_t* zero,
                 size_t* norm, size_t* sink, size_t* extra) {
  *extra = (size_t)(dv.n_vec * dv.extra_bytes);
  *codes = (size_t)(dv.n_vec * dv.code_bytes);
  *scale = (size_t)(dv.n_vec * dv.ngroups * 2);
  *zero = *scale;
  *norm = cfg->quant == KVQ_Q_LLOYD ? (size_t)(dv.n_vec * 4) : 0;
  *sink = cfg->n_sink > 0 ? (size_t)(cfg->rows * (int64_t)cfg->n_sink * cfg->heads * cfg->head_dim * 2) : 0;
}

bool sinks_in_range(const kvq_config* cfg) {
  return cfg->n_sink > 0 && cfg->tokens > 0 && cfg->pos_offset < cfg->n_sink;
}

kvq_status check_planes(const kvq_config* cfg, const Derived& dv, const kvq_planes* pl) {
  if (!pl) return fail(KVQ_ERR_NULL, "planes is NULL");
  if (dv.n_vec == 0) return KVQ_OK;
  if (!pl->codes) return fail(KVQ_ERR_NULL, "codes plane is NULL");
  if (!aligned16(pl->codes)) return fail(KVQ_ERR_ALIGN, "codes plane not 16-byte aligned");
  if (cfg->quant == KVQ_Q_MINMAX) {
    if (!pl->scale || !pl->zero) return fail(KVQ_ERR_NULL, "scale/zero plane is NULL");
    if (!aligned16(pl->scale) || !aligned16(pl->zero)) return fail(KVQ_ERR_ALIGN, "scale/zero plane not 16-byte aligned");
  } else {
    if (!pl->norm) return fail(KVQ_ERR_NULL, "norm plane is NULL");
    if (!aligned16(pl->norm)) return fail(KVQ_ERR_ALIGN, "norm plane not 16-byte aligned");
  }
  if (dv.extra_bytes) {
    if (!pl->extra) return fail(KVQ_ERR_NULL, "extra plane is NULL (dynamic codebook)");
    if (!aligned16(pl->extra)) return fail(KVQ_ERR_ALIGN, "extra plane not 16-byte aligned");
  }
  if (sinks_in_range(cfg)) {
    if (!pl->sink) return fail(KVQ_ERR_NULL, "sink plane is NULL");
    if (!aligned16(pl->sink)) return fail(KVQ_ERR_ALIGN, "sink plane not 16-byte aligned");
  }
  return KVQ_OK;
}

// Work decomposition: an item is (tile of VPW consecutive (token, head) columns, row);
// the launcher groups items into tasks, one wave each (runs of rows of one tile in the
// encoder, runs of tiles of one row in the decoder).
void plan_work(const kvq_config* cfg, kvq::CodecArgs* a) {
  const int vpw = cfg->head_dim == 128 ? 16 : 8;
  const int64_t ncols = cfg->tokens * cfg->heads;
  a->n_tiles = (ncols + vpw - 1) / vpw;
  a->n_items = cfg->rows * a->n_tiles;
  a->div_heads = kvq::make_fastdiv((uint32_t)std::max<int64_t>(cfg->heads, 1));
}

void fill_args(const kvq_config* cfg, const Derived& dv, kvq::CodecArgs* a) {
  memset(a, 0, sizeof *a);
  a->rows = cfg->rows;
  a->tokens = cfg->tokens;
  a->heads = cfg->heads;
  a->sr = dv.sr;
  a->st = dv.st;
  a->sh = dv.sh;
  a->pos_offset = cfg->pos_offset;
  a->rope = cfg->rope;
  a->rope_log2_base = cfg->rope ? log2(cfg->rope_base) : 0.0;
  a->group_log2 = cfg->quant == KVQ_Q_MINMAX ? ilog2(cfg->group_size) : 0;
  a->n_sink = cfg->n_sink;
  a->use_perm = cfg->perm ? 1 : 0;
  if (cfg->perm)
    for (int64_t i = 0; i < cfg->head_dim; ++i) a->perm[i] = (uint8_t)cfg->perm[i];
  if (cfg->rot == KVQ_ROT_SO4) memcpy(a->quat, cfg->quat, sizeof(float) * cfg->head_dim / 4 * 8);
  if (cfg->rot == KVQ_ROT_ROTOR) {
    // the kernels' rotor parameters: rotor b at quat[4 b], then the tail's (cos, sin)
    const int64_t nb = cfg->head_dim / 3;
    memcpy(a->quat, cfg->rotor_quat, sizeof(float) * 4 * nb);
    a->quat[4 * nb] = (float)cos(cfg->rotor_tail);
    a->quat[4 * nb + 1] = (float)sin(cfg->rotor_tail);
  }
  if (cfg->quant == KVQ_Q_LLOYD) memcpy(a->codebook, cfg->codebook, sizeof(float) * (1 << cfg->bits));
  if (dv.extra_bytes) {
    a->dyn = 1;
    memcpy(a->chan_scale, cfg->chan_scale, sizeof(float) * cfg->head_dim);
    memcpy(a->codebook_wide, cfg->codebook_wide, sizeof(float) * (2 << cfg->bits));
    int k = 0;
    for (int64_t j = 0; j < cfg->head_dim; ++j) a->wide_rank[j] = cfg->chan_wide[j] ? (uint8_t)k++ : 0xff;
  }
  a->rot_matrix = cfg->rot == KVQ_ROT_DENSE ? cfg->rot_matrix : nullptr;
}

// ---- Lloyd-Max (host, double precision) ----
double npdf(double x) { return isinf(x) ? 0.0 : exp(-0.5 * x * x) * 0.3989422804014327; }
// upper tail Q(x) = P(X > x)
double ntail(double x) { return 0.5 * erfc(x * 0.7071067811865476); }

}  // namespace

extern "C" {

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

kvq_status kvq_validate(const kvq_config* cfg) {
  Derived dv;
  kvq_status st = check_config(cfg, &dv);
  return st == KVQ_OK ? ok() : st;
}

kvq_status kvq_packed_sizes(const kvq_config* cfg, size_t* codes, size_t* scale, size_t* zero, size_t* norm,
                            size_t* sink, size_t* extra) {
  Derived dv;
  kvq_status st = check_config(cfg, &dv);
  if (st != KVQ_OK) return st;
  if (!codes || !scale || !zero || !norm || !sink || !extra) return fail(KVQ_ERR_NULL, "size output pointer is NULL");
  plane_sizes(cfg, dv, codes, scale, zero, norm, sink, extra);
  return ok();
}

namespace {
// the dense rotation's codec: head_dim 128, no dynamic codebook
kvq_status check_dense(const kvq_config* cfg) {
  if (cfg->head_dim != 128) return fail(KVQ_ERR_UNSUPPORTED, "dense rotation: head_dim 128 only");
  if (cfg->chan_scale) return fail(KVQ_ERR_UNSUPPORTED, "dense rotation: no dynamic codebook");
  return KVQ_OK;
}
}  // namespace

kvq_status kvq_encode(const kvq_config* cfg, const void* x, const kvq_planes* out, void* stream) {
  Derived dv;
  kvq_status st = check_config(cfg, &dv);
  if (st != KVQ_OK) return st;
  if (cfg->rot == KVQ_ROT_DENSE && (st = check_dense(cfg)) != KVQ_OK) return st;
  if ((st = check_planes(cfg, dv, out)) != KVQ_OK) return st;
  if (dv.n_vec == 0) return ok();
  if (!x) return fail(KVQ_ERR_NULL, "x is NULL");
  if (!aligned16(x)) return fail(KVQ_ERR_ALIGN, "x not 16-byte aligned");
  kvq::CodecArgs a;
  fill_args(cfg, dv, &a);
  a.x = x;
  a.codes = static_cast<uint8_t*>(out->codes);
  a.scale = static_cast<uint16_t*>(out->scale);
  a.zero = static_cast<uint16_t*>(out->zero);
  a.norm = static_cast<float*>(out->norm);
  a.sink = static_cast<uint16_t*>(out->sink);
  a.extra = static_cast<uint8_t*>(out->extra);
  plan_work(cfg, &a);
  const bool d128 = cfg->head_dim == 128;
  int err;
  if (cfg->rot == KVQ_ROT_DENSE) {
    err = kvq::launch_encode_dense(cfg->dtype, cfg->bits, cfg->quant, a, stream);
  } else {
    switch (cfg->dtype) {
      case KVQ_F16:
        err = (d128 ? kvq::launch_encode_f16_d128 : kvq::launch_encode_f16_d256)(cfg->bits, cfg->rot, cfg->quant, a, stream);
        break;
      case KVQ_BF16:
        err = (d128 ? kvq::launch_encode_bf16_d128 : kvq::launch_encode_bf16_d256)(cfg->bits, cfg->rot, cfg->quant, a, stream);
        break;
      default:
        err = (d128 ? kvq::launch_encode_f32_d128 : kvq::launch_encode_f32_d256)(cfg->bits, cfg->rot, cfg->quant, a, stream);
        break;
    }
  }
  if (err != 0) return fail(KVQ_ERR_DEVICE, "encode launch failed: %s", kvq::device_error_string(err));
  return ok();
}

kvq_status kvq_append(const kvq_config* cfg, const void* x, const int64_t* positions, const kvq_planes* cache,
                      void* stream) {
  Derived dv;
  kvq_status st = check_config(cfg, &dv);  // cfg describes the cache: tokens = slots per row
  if (st != KVQ_OK) return st;
  if (cfg->rot == KVQ_ROT_DENSE || cfg->rot == KVQ_ROT_ROTOR)
    return fail(KVQ_ERR_UNSUPPORTED, "dense and rotor rotations: no append (encode the batch)");
  if (!cache) return fail(KVQ_ERR_NULL, "cache planes is NULL");
  if (dv.n_vec == 0) return ok();
  if ((st = check_planes(cfg, dv, cache)) != KVQ_OK) return st;
  // a sink plane is needed whenever some slot of the cache is a sink position
  if (cfg->n_sink > 0 && cfg->pos_offset < cfg->n_sink && !cache->sink)
    return fail(KVQ_ERR_NULL, "sink plane is NULL");
  if (!x) return fail(KVQ_ERR_NULL, "x is NULL");
  if (!positions) return fail(KVQ_ERR_NULL, "positions is NULL");
  if (!aligned16(x)) return fail(KVQ_ERR_ALIGN, "x not 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(positions) & 7u) != 0) return fail(KVQ_ERR_ALIGN, "positions not 8-byte aligned");
  kvq::CodecArgs a;
  fill_args(cfg, dv, &a);
  // the input is one vector per (row, head): [R, H, D] with the row and head strides
  const bool contiguous = cfg->stride_r == 0 && cfg->stride_t == 0 && cfg->stride_h == 0;
  a.tokens = 1;
  a.sr = contiguous ? cfg->heads * cfg->head_dim : cfg->stride_r;
  a.st = 0;
  a.sh = contiguous ? cfg->head_dim : cfg->stride_h;
  a.cap = cfg->tokens;
  a.row_pos = positions;
  a.x = x;
  a.codes = static_cast<uint8_t*>(cache->codes);
  a.scale = static_cast<uint16_t*>(cache->scale);
  a.zero = static_cast<uint16_t*>(cache->zero);
  a.norm = static_cast<float*>(cache->norm);
  a.sink = static_cast<uint16_t*>(cache->sink);
  a.extra = static_cast<uint8_t*>(cache->extra);
  const int vpw = cfg->head_dim == 128 ? 16 : 8;
  a.n_tiles = (cfg->heads + vpw - 1) / vpw;
  a.n_items = cfg->rows * a.n_tiles;
  a.div_heads = kvq::make_fastdiv((uint32_t)std::max<int64_t>(cfg->heads, 1));
  const bool d128 = cfg->head_dim == 128;
  int err;
  switch (cfg->dtype) {
    case KVQ_F16:
      err = (d128 ? kvq::launch_encode_f16_d128 : kvq::launch_encode_f16_d256)(cfg->bits, cfg->rot, cfg->quant, a, stream);
      break;
    case KVQ_BF16:
      err = (d128 ? kvq::launch_encode_bf16_d128 : kvq::launch_encode_bf16_d256)(cfg->bits, cfg->rot, cfg->quant, a, stream);
      break;
    default:
      err = (d128 ? kvq::launch_encode_f32_d128 : kvq::launch_encode_f32_d256)(cfg->bits, cfg->rot, cfg->quant, a, stream);
      break;
  }
  if (err != 0) return fail(KVQ_ERR_DEVICE, "append launch failed: %s", kvq::device_error_string(err));
  return ok();
}

kvq_status kvq_decode(const kvq_config* cfg, const kvq_planes* in, void* y, int32_t y_dtype, void* stream) {
  Derived dv;
  kvq_status st = check_config(cfg, &dv);
  if (st != KVQ_OK) return st;
  if (cfg->rot == KVQ_ROT_DENSE && (st = check_dense(cfg)) != KVQ_OK) return st;
  if (y_dtype < KVQ_F16 || y_dtype > KVQ_F32) return fail(KVQ_ERR_ROT, "unknown output dtype %d", y_dtype);
  if ((st = check_planes(cfg, dv, in)) != KVQ_OK) return st;
  if (dv.n_vec == 0) return ok();
  if (!y) return fail(KVQ_ERR_NULL, "y is NULL");
  if (!aligned16(y)) return fail(KVQ_ERR_ALIGN, "y not 16-byte aligned");
  kvq::CodecArgs a;
  fill_args(cfg, dv, &a);
  a.y = y;
  a.codes = static_cast<uint8_t*>(in->codes);
  a.scale = static_cast<uint16_t*>(in->scale);
  a.zero = static_cast<uint16_t*>(in->zero);
  a.norm = static_cast<float*>(in->norm);
  a.sink = static_cast<uint16_t*>(in->sink);
  a.extra = static_cast<uint8_t*>(in->extra);
  plan_work(cfg, &a);
  const bool d128 = cfg->head_dim == 128;
  int err;
  if (cfg->rot == KVQ_ROT_DENSE) {
    err = kvq::launch_decode_dense(y_dtype, cfg->bits, cfg->quant, a, stream);
  } else {
    switch (y_dtype) {
      case KVQ_F16:
        err = (d128 ? kvq::launch_decode_f16_d128 : kvq::launch_decode_f16_d256)(cfg->bits, cfg->rot, cfg->quant, a, stream);
        break;
      case KVQ_BF16:
        err = (d128 ? kvq::launch_decode_bf16_d128 : kvq::launch_decode_bf16_d256)(cfg->bits, cfg->rot, cfg->quant, a, stream);
        break;
      default:
        err = (d128 ? kvq::launch_decode_f32_d128 : kvq::launch_decode_f32_d256)(cfg->bits, cfg->rot, cfg->quant, a, stream);
        break;
    }
  }
  if (err != 0) return fail(KVQ_ERR_DEVICE, "decode launch failed: %s", kvq::device_error_string(err));
  return ok();
}

namespace {
// The configurations decode-step attention supports, the pass that serves them, and the
// workspace it needs.  cfg_v NULL stands for a V cache configured like K.  The matrix-core
// passes (fast) take head_dim 128, Walsh-Hadamard, K and V of equal bits (2 or 4) and group,
// slot t = position t and up to 4 query heads per KV head; the general pass takes the rest.
kvq_status check_attend(const kvq_config* cfg_k, const kvq_config* cfg_v, int64_t q_heads, size_t* ws_bytes,
                        kvq::AttendArgs* a, bool* fast_out) {
  Derived dk, dv;
  kvq_status st = check_config(cfg_k, &dk);
  if (st != KVQ_OK) return st;
  if (cfg_v) {
    if ((st = check_config(cfg_v, &dv)) != KVQ_OK) return st;
    if (cfg_v->rows != cfg_k->rows || cfg_v->tokens != cfg_k->tokens || cfg_v->heads != cfg_k->heads ||
        cfg_v->head_dim != cfg_k->head_dim || cfg_v->n_sink != cfg_k->n_sink ||
        cfg_v->pos_offset != cfg_k->pos_offset || cfg_v->rot != cfg_k->rot || cfg_v->quant != cfg_k->quant)
      return fail(KVQ_ERR_SHAPE, "the K and V caches must share rows, slots, heads, head_dim, sinks, pos_offset, "
                                 "rotation and quantizer");
  }
  const kvq_config* cv = cfg_v ? cfg_v : cfg_k;
  const int64_t d = cfg_k->head_dim;
  if ((d != 128 && d != 256) || (cfg_k->rot != KVQ_ROT_FWHT && cfg_k->rot != KVQ_ROT_NONE) ||
      cfg_k->quant != KVQ_Q_MINMAX)
    return fail(KVQ_ERR_UNSUPPORTED, "attention supports head_dim 128 or 256, Walsh-Hadamard or no rotation, "
                                     "min-max codes");
  if (cfg_k->n_sink > 64) return fail(KVQ_ERR_UNSUPPORTED, "attention supports at most 64 sink positions");
  if (cfg_k->heads <= 0 || q_heads <= 0 || q_heads % cfg_k->heads != 0)
    return fail(KVQ_ERR_SHAPE, "q_heads must be a positive multiple of heads");
  const int64_t qg = q_heads / cfg_k->heads;
  if (qg != 1 && qg != 2 && qg != 4 && qg != 8)
    return fail(KVQ_ERR_UNSUPPORTED, "attention supports 1, 2, 4 or 8 query heads per KV head");
  const bool fast = d == 128 && cfg_k->rot == KVQ_ROT_FWHT && cv->bits == cfg_k->bits &&
                    (cfg_k->bits == 2 || cfg_k->bits == 4) && cv->group_size == cfg_k->group_size &&
                    cfg_k->group_size <= 128 && cfg_k->pos_offset == 0 && qg <= 4;
  int32_t nc = 1, ct = 8;
  const bool mma_blk = fast && cfg_k->group_size == 128 && cfg_k->heads % 4 == 0;
  kvq::attend_chunks(cfg_k->rows, cfg_k->heads, cfg_k->tokens, mma_blk, &nc, &ct);
  int64_t nq = 0, tmp = 0;
  if (!mul_ok(cfg_k->rows, q_heads, &nq) || !mul_ok(nq, (int64_t)nc * (d + 2) + d, &tmp) || tmp > (int64_t(1) << 40))
    return fail(KVQ_ERR_SHAPE, "attention workspace too large");
  const size_t q_bytes = (size_t)(nq * d * 4 + 255) / 256 * 256;
  *ws_bytes = q_bytes + (size_t)nq * (size_t)nc * (size_t)(d + 2) * 4;
  if (fast_out) *fast_out = fast;
  if (a) {
    memset(a, 0, sizeof *a);
    a->rows = cfg_k->rows;
    a->tokens = cfg_k->tokens;
    a->heads = cfg_k->heads;
    a->q_heads = q_heads;
    a->group_log2 = ilog2(cfg_k->group_size);
    a->v_group_log2 = ilog2(cv->group_size);
    a->n_sink = cfg_k->n_sink;
    a->n_chunks = nc;
    a->chunk = ct;
    a->rot = cfg_k->rot == KVQ_ROT_FWHT ? 1 : 0;
    // slots 0 .. sink_slots - 1 hold positions pos_offset .. below n_sink
    const int64_t ss = (int64_t)cfg_k->n_sink - cfg_k->pos_offset;
    a->sink_slots = (int32_t)(ss <= 0 ? 0 : (ss < cfg_k->tokens ? ss : cfg_k->tokens));
    a->sink_base = a->sink_slots > 0 ? (int32_t)cfg_k->pos_offset : 0;
    a->use_perm_k = cfg_k->perm ? 1 : 0;
    if (cfg_k->perm)
      for (int64_t i = 0; i < d; ++i) a->perm_k[i] = (uint8_t)cfg_k->perm[i];
    a->use_perm_v = cv->perm ? 1 : 0;
    if (cv->perm)
      for (int64_t i = 0; i < d; ++i) a->perm_v[i] = (uint8_t)cv->perm[i];
  }
  return KVQ_OK;
}
}  // namespace

kvq_status kvq_attend_workspace_size(const kvq_config* cfg_k, const kvq_config* cfg_v, int64_t q_heads,
                                     size_t* bytes) {
  if (!bytes) return fail(KVQ_ERR_NULL, "bytes is NULL");
  kvq_status st = check_attend(cfg_k, cfg_v, q_heads, bytes, nullptr, nullptr);
  return st == KVQ_OK ? ok() : st;
}

namespace {
// kvq_attend and kvq_attend_noalloc: every check, then the launches.  With workspace NULL and
// use_scratch set, the workspace is the library's static device array (looked up only after
// every check has passed, so an error return has made no HIP call).
kvq_status attend_impl(const kvq_config* cfg_k, const kvq_planes* k, const kvq_config* cfg_v, const kvq_planes* v,
                       const float* q, int64_t q_heads, const int32_t* lengths, float scale, float* out,
                       void* workspace, size_t workspace_bytes, bool use_scratch, void* stream) {
  if (!cfg_v) return fail(KVQ_ERR_NULL, "cfg_v is NULL");
  size_t need = 0;
  bool fast = false;
  kvq::AttendArgs a;
  kvq_status st = check_attend(cfg_k, cfg_v, q_heads, &need, &a, &fast);
  if (st != KVQ_OK) return st;
  if (!isfinite(scale)) return fail(KVQ_ERR_PARAM, "scale must be finite");
  Derived dk, dv;
  (void)check_config(cfg_k, &dk);  // both already accepted above; this fills the derived sizes
  (void)check_config(cfg_v, &dv);
  if (!k || !v) return fail(KVQ_ERR_NULL, "planes is NULL");
  if (cfg_k->rows == 0) return ok();
  // (a cache with no slot still runs: every output row is then zero)
  if ((st = check_planes(cfg_k, dk, k)) != KVQ_OK) return st;
  if ((st = check_planes(cfg_v, dv, v)) != KVQ_OK) return st;
  if (a.sink_slots > 0 && (!k->sink || !v->sink)) return fail(KVQ_ERR_NULL, "sink plane is NULL");
  if (!q || !out) return fail(KVQ_ERR_NULL, "q or out is NULL");
  if (!use_scratch && !workspace) return fail(KVQ_ERR_NULL, "workspace is NULL");
  if (!aligned16(q) || !aligned16(out) || (!use_scratch && !aligned16(workspace)))
    return fail(KVQ_ERR_ALIGN, "q, out and workspace must be 16-byte aligned");
  if (lengths && (reinterpret_cast<uintptr_t>(lengths) & 3u)) return fail(KVQ_ERR_ALIGN, "lengths not 4-byte aligned");
  if (use_scratch) {
    if (need > kvq::kAttendScratchBytes)
      return fail(KVQ_ERR_SHAPE, "kvq_attend_noalloc: this cache and query-head count need %zu bytes of workspace, "
                                 "above its fixed %zu (use kvq_attend with a workspace)",
                  need, kvq::kAttendScratchBytes);
    if (const int e = kvq::attend_scratch(&workspace))
      return fail(KVQ_ERR_DEVICE, "kvq_attend_noalloc: device workspace lookup failed: %s", kvq::device_error_string(e));
  } else if (workspace_bytes < need) {
    return fail(KVQ_ERR_SHAPE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  }
  a.k_codes = static_cast<const uint8_t*>(k->codes);
  a.k_scale = static_cast<const uint16_t*>(k->scale);
  a.k_zero = static_cast<const uint16_t*>(k->zero);
  a.k_sink = static_cast<const uint16_t*>(k->sink);
  a.v_codes = static_cast<const uint8_t*>(v->codes);
  a.v_scale = static_cast<const uint16_t*>(v->scale);
  a.v_zero = static_cast<const uint16_t*>(v->zero);
  a.v_sink = static_cast<const uint16_t*>(v->sink);
  a.q = q;
  a.out = out;
  const int64_t d = cfg_k->head_dim;
  a.qrot = static_cast<float*>(workspace);
  a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + (size_t)(a.rows * q_heads * d * 4 + 255) / 256 * 256);
  a.lengths = lengths;
  a.scale = scale;
  const int qg = (int)(q_heads / cfg_k->heads);
  int err;
  if (fast) {
    err = kvq::launch_attend(cfg_k->bits, qg, a, stream);
  } else {
    const int kb = cfg_k->bits, vb = cfg_v->bits;
    if (d == 128)
      err = (kb == 2 ? kvq::launch_attend_gen_d128_k2 : kb == 3 ? kvq::launch_attend_gen_d128_k3
                                                                 : kvq::launch_attend_gen_d128_k4)(vb, qg, a, stream);
    else
      err = (kb == 2 ? kvq::launch_attend_gen_d256_k2 : kb == 3 ? kvq::launch_attend_gen_d256_k3
                                                                 : kvq::launch_attend_gen_d256_k4)(vb, qg, a, stream);
  }
  if (err != 0) return fail(KVQ_ERR_DEVICE, "attention launch failed: %s", kvq::device_error_string(err));
  return ok();
}
}  // namespace

kvq_status kvq_attend(const kvq_config* cfg_k, const kvq_planes* k, const kvq_config* cfg_v, const kvq_planes* v,
                      const float* q, int64_t q_heads, const int32_t* lengths, float scale, float* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return attend_impl(cfg_k, k, cfg_v, v, q, q_heads, lengths, scale, out, workspace, workspace_bytes, false, stream);
}

kvq_status kvq_attend_noalloc(const kvq_config* cfg_k, const kvq_planes* k, const kvq_config* cfg_v,
                              const kvq_planes* v, const float* q, int64_t q_heads, const int32_t* lengths, float scale,
                              float* out, void* stream) {
  return attend_impl(cfg_k, k, cfg_v, v, q, q_heads, lengths, scale, out, nullptr, 0, true, stream);
}

size_t kvq_attend_noalloc_max_workspace(void) { return kvq::kAttendScratchBytes; }

namespace {
// the calibration calls read x exactly as kvq_encode does (shape, dtype, strides, RoPE,
// positions and sinks from cfg)
void fill_calib(const kvq_config* cfg, const Derived& dv, const void* x, kvq::CalibArgs* a) {
  memset(a, 0, sizeof *a);
  a->x = x;
  a->rows = cfg->rows;
  a->tokens = cfg->tokens;
  a->heads = cfg->heads;
  a->head_dim = cfg->head_dim;
  a->sr = dv.sr;
  a->st = dv.st;
  a->sh = dv.sh;
  a->pos_offset = cfg->pos_offset;
  a->rope = cfg->rope;
  a->rope_log2_base = cfg->rope ? log2(cfg->rope_base) : 0.0;
  a->n_sink = cfg->n_sink;
  a->dtype = cfg->dtype;
  a->tpw = kvq::calib_tokens_per_wave(cfg->rows, cfg->tokens);
  a->n_waves = cfg->rows * ((cfg->tokens + a->tpw - 1) / a->tpw);
}
}  // namespace

kvq_status kvq_channel_stats_workspace_size(const kvq_config* cfg, size_t* bytes) {
  if (!bytes) return fail(KVQ_ERR_NULL, "bytes is NULL");
  Derived dv;
  kvq_status st = check_config(cfg, &dv);
  if (st != KVQ_OK) return st;
  kvq::CalibArgs a;
  fill_calib(cfg, dv, nullptr, &a);
  *bytes = (size_t)a.n_waves * (size_t)cfg->head_dim * sizeof(double);
  return ok();
}

kvq_status kvq_channel_stats(const kvq_config* cfg, const void* x, double* stats, void* workspace,
                             size_t workspace_bytes, void* stream) {
  Derived dv;
  kvq_status st = check_config(cfg, &dv);
  if (st != KVQ_OK) return st;
  if (!stats) return fail(KVQ_ERR_NULL, "stats is NULL");
  if (reinterpret_cast<uintptr_t>(stats) & 7u) return fail(KVQ_ERR_ALIGN, "stats not 8-byte aligned");
  kvq::CalibArgs a;
  fill_calib(cfg, dv, x, &a);
  const size_t need = (size_t)a.n_waves * (size_t)cfg->head_dim * sizeof(double);
  if (need > 0) {
    if (!x) return fail(KVQ_ERR_NULL, "x is NULL");
    if (!aligned16(x)) return fail(KVQ_ERR_ALIGN, "x not 16-byte aligned");
    if (!workspace) return fail(KVQ_ERR_NULL, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) & 7u) return fail(KVQ_ERR_ALIGN, "workspace not 8-byte aligned");
    if (workspace_bytes < need) return fail(KVQ_ERR_SHAPE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  }
  a.part = static_cast<double*>(workspace);
  a.stats = stats;
  if (a.n_waves > (int64_t(1) << 33)) return fail(KVQ_ERR_SHAPE, "calibration slice too large");
  const int err = kvq::launch_channel_stats(a, stream);
  if (err != 0) return fail(KVQ_ERR_DEVICE, "channel statistics launch failed: %s", kvq::device_error_string(err));
  return ok();
}

kvq_status kvq_rotated_moments(const kvq_config* cfg, const void* x, double* moments, void* workspace,
                               size_t workspace_bytes, void* stream) {
  Derived dv;
  kvq_status st = check_config(cfg, &dv);
  if (st != KVQ_OK) return st;
  if (cfg->quant != KVQ_Q_LLOYD) return fail(KVQ_ERR_PARAM, "rotated moments belong to the Lloyd-Max path (quant)");
  if (cfg->rot == KVQ_ROT_ROTOR) return fail(KVQ_ERR_UNSUPPORTED, "rotated moments: no rotor rotation");
  if (!moments) return fail(KVQ_ERR_NULL, "moments is NULL");
  if (reinterpret_cast<uintptr_t>(moments) & 7u) return fail(KVQ_ERR_ALIGN, "moments not 8-byte aligned");
  kvq::CalibArgs a;
  fill_calib(cfg, dv, x, &a);
  const size_t need = (size_t)a.n_waves * (size_t)cfg->head_dim * sizeof(double);
  if (need > 0) {
    if (!x) return fail(KVQ_ERR_NULL, "x is NULL");
    if (!aligned16(x)) return fail(KVQ_ERR_ALIGN, "x not 16-byte aligned");
    if (!workspace) return fail(KVQ_ERR_NULL, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) & 7u) return fail(KVQ_ERR_ALIGN, "workspace not 8-byte aligned");
    if (workspace_bytes < need) return fail(KVQ_ERR_SHAPE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  }
  if (a.n_waves > (int64_t(1) << 33)) return fail(KVQ_ERR_SHAPE, "calibration slice too large");
  a.part = static_cast<double*>(workspace);
  a.stats = moments;
  a.rot = cfg->rot;
  a.rot_matrix = cfg->rot == KVQ_ROT_DENSE ? cfg->rot_matrix : nullptr;
  a.use_perm = cfg->perm ? 1 : 0;
  if (cfg->perm)
    for (int64_t i = 0; i < cfg->head_dim; ++i) a.perm[i] = (uint8_t)cfg->perm[i];
  if (cfg->rot == KVQ_ROT_SO4) memcpy(a.quat, cfg->quat, sizeof(float) * cfg->head_dim / 4 * 8);
  const int err = kvq::launch_rotated_moments(a, stream);
  if (err != 0) return fail(KVQ_ERR_DEVICE, "rotated moments launch failed: %s", kvq::device_error_string(err));
  return ok();
}

kvq_status kvq_dynamic_codebook(const double* moments, int64_t head_dim, int32_t bits, float* chan_scale,
                                uint8_t* chan_wide, float* codebook, float* codebook_wide) {
  if (!moments || !chan_scale || !chan_wide || !codebook || !codebook_wide)
    return fail(KVQ_ERR_NULL, "an argument of kvq_dynamic_codebook is NULL");
  if (head_dim != 128 && head_dim != 256)
    return fail(KVQ_ERR_UNSUPPORTED, "head_dim %lld (supported: 128, 256)", (long long)head_dim);
  if (bits < 2 || bits > 4) return fail(KVQ_ERR_BITS, "bits %d (supported: 2, 3, 4)", bits);
  const int d = (int)head_dim;
  for (int j = 0; j < d; ++j)
    if (!(isfinite(moments[j]) && moments[j] > 0.0))
      return fail(KVQ_ERR_PARAM, "moments[%d] must be finite and > 0", j);
  // the KL-closest zero-mean Gaussian to a channel is the one with its second moment
  for (int j = 0; j < d; ++j) chan_scale[j] = (float)sqrt(moments[j]);
  // wide channels: the d/16 largest scales (equal scales in increasing channel order)
  int order[kvq::kMaxHeadDim];
  for (int j = 0; j < d; ++j) order[j] = j;
  std::stable_sort(order, order + d, [&](int i, int j) { return moments[i] > moments[j]; });
  for (int j = 0; j < d; ++j) chan_wide[j] = 0;
  for (int k = 0; k < d / 16; ++k) chan_wide[order[k]] = 1;
  kvq_status st = kvq_lloyd_max_gaussian(bits, 1.0, codebook);
  if (st != KVQ_OK) return st;
  return kvq_lloyd_max_gaussian(bits + 1, 1.0, codebook_wide);
}

kvq_status kvq_outlier_perm(const double* stats, int64_t head_dim, int32_t group_size, uint16_t* perm) {
  if (!stats || !perm) return fail(KVQ_ERR_NULL, "stats or perm is NULL");
  if (head_dim != 128 && head_dim != 256)
    return fail(KVQ_ERR_UNSUPPORTED, "head_dim %lld (supported: 128, 256)", (long long)head_dim);
  if (!(group_size == 32 || group_size == 64 || group_size == 128 || group_size == 256) || group_size > head_dim)
    return fail(KVQ_ERR_GROUP, "group_size %d (32, 64, 128 or 256, at most head_dim)", group_size);
  const int d = (int)head_dim;
  for (int c = 0; c < d; ++c)
    if (!isfinite(stats[c])) return fail(KVQ_ERR_PARAM, "stats[%d] is not finite", c);
  // channels by decreasing statistic, equal statistics in increasing channel order
  int order[kvq::kMaxHeadDim];
  for (int c = 0; c < d; ++c) order[c] = c;
  std::stable_sort(order, order + d, [&](int i, int j) { return stats[i] > stats[j]; });
  const int k = d / group_size;
  bool top[kvq::kMaxHeadDim] = {false};
  for (int a = 0; a < k; ++a) {
    perm[a * group_size] = (uint16_t)order[a];
    top[order[a]] = true;
  }
  // the other channels, in increasing order, fill the positions that are not multiples of G
  int j = 0;
  for (int c = 0; c < d; ++c) {
    if (top[c]) continue;
    while (j % group_size == 0) ++j;
    perm[j++] = (uint16_t)c;
  }
  return ok();
}

kvq_status kvq_detect_sinks(const kvq_config* cfg, const void* x, double lambda, double* norms, uint8_t* flags,
                            int32_t* counts, int32_t* prefix, double* medians, void* stream) {
  Derived dv;
  kvq_status st = check_config(cfg, &dv);
  if (st != KVQ_OK) return st;
  if (!(isfinite(lambda) && lambda >= 0.0)) return fail(KVQ_ERR_PARAM, "lambda must be finite and >= 0");
  if (cfg->rows == 0) return ok();
  if (!counts || !prefix || !medians) return fail(KVQ_ERR_NULL, "counts, prefix or medians is NULL");
  if ((reinterpret_cast<uintptr_t>(counts) & 3u) || (reinterpret_cast<uintptr_t>(prefix) & 3u) ||
      (reinterpret_cast<uintptr_t>(medians) & 7u))
    return fail(KVQ_ERR_ALIGN, "counts, prefix (4 bytes) or medians (8 bytes) misaligned");
  if (cfg->tokens > 0) {
    if (!x || !norms || !flags) return fail(KVQ_ERR_NULL, "x, norms or flags is NULL");
    if (!aligned16(x)) return fail(KVQ_ERR_ALIGN, "x not 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(norms) & 7u) return fail(KVQ_ERR_ALIGN, "norms not 8-byte aligned");
  }
  kvq::CalibArgs a;
  fill_calib(cfg, dv, x, &a);
  a.lambda = lambda;
  a.norms = norms;
  a.flags = flags;
  a.counts = counts;
  a.prefix = prefix;
  a.medians = medians;
  if (cfg->rows > 0x7fffffff || cfg->rows * cfg->tokens > (int64_t(1) << 33))
    return fail(KVQ_ERR_SHAPE, "calibration slice too large");
  const int err = kvq::launch_detect_sinks(a, stream);
  if (err != 0) return fail(KVQ_ERR_DEVICE, "sink detection launch failed: %s", kvq::device_error_string(err));
  return ok();
}

namespace {
kvq_status check_entropy(const kvq_config* cfg, int64_t q_heads, size_t* ws_bytes, kvq::EntropyArgs* a) {
  Derived dv;
  kvq_status st = check_config(cfg, &dv);
  if (st != KVQ_OK) return st;
  if (cfg->rot != KVQ_ROT_FWHT || cfg->quant != KVQ_Q_MINMAX)
    return fail(KVQ_ERR_UNSUPPORTED, "attention entropy reads Walsh-Hadamard + min-max caches");
  if (cfg->pos_offset != 0) return fail(KVQ_ERR_UNSUPPORTED, "attention entropy needs pos_offset 0 (slot = position)");
  if (cfg->heads <= 0 || q_heads <= 0 || q_heads % cfg->heads != 0)
    return fail(KVQ_ERR_SHAPE, "q_heads must be a positive multiple of heads");
  const int64_t qg = q_heads / cfg->heads;
  if (qg != 1 && qg != 2 && qg != 4 && qg != 8)
    return fail(KVQ_ERR_UNSUPPORTED, "attention entropy supports 1, 2, 4 or 8 query heads per KV head");
  int32_t nc = 1, ct = 8;
  kvq::attend_chunks(cfg->rows, cfg->heads, cfg->tokens, false, &nc, &ct);
  int64_t nq = 0, tmp = 0;
  if (!mul_ok(cfg->rows, q_heads, &nq) || !mul_ok(nq, (int64_t)nc * 4 + cfg->head_dim, &tmp) || tmp > (int64_t(1) << 40))
    return fail(KVQ_ERR_SHAPE, "entropy workspace too large");
  const size_t q_bytes = (size_t)(nq * cfg->head_dim * 4 + 255) / 256 * 256;
  *ws_bytes = q_bytes + (size_t)nq * (size_t)nc * 16;
  if (a) {
    memset(a, 0, sizeof *a);
    a->rows = cfg->rows;
    a->tokens = cfg->tokens;
    a->heads = cfg->heads;
    a->q_heads = q_heads;
    a->head_dim = cfg->head_dim;
    a->bits = cfg->bits;
    a->group_log2 = ilog2(cfg->group_size);
    a->n_sink = cfg->n_sink;
    a->n_chunks = nc;
    a->chunk = ct;
    a->use_perm = cfg->perm ? 1 : 0;
    if (cfg->perm)
      for (int64_t i = 0; i < cfg->head_dim; ++i) a->perm[i] = (uint8_t)cfg->perm[i];
  }
  return KVQ_OK;
}
}  // namespace

kvq_status kvq_attention_entropy_workspace_size(const kvq_config* cfg_k, int64_t q_heads, size_t* bytes) {
  if (!bytes) return fail(KVQ_ERR_NULL, "bytes is NULL");
  kvq_status st = check_entropy(cfg_k, q_heads, bytes, nullptr);
  return st == KVQ_OK ? ok() : st;
}

kvq_status kvq_attention_entropy(const kvq_config* cfg_k, const kvq_planes* k, const float* q, int64_t q_heads,
                                 const int32_t* lengths, float scale, float* entropy, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  size_t need = 0;
  kvq::EntropyArgs a;
  kvq_status st = check_entropy(cfg_k, q_heads, &need, &a);
  if (st != KVQ_OK) return st;
  if (!isfinite(scale)) return fail(KVQ_ERR_PARAM, "scale must be finite");
  if (!k) return fail(KVQ_ERR_NULL, "planes is NULL");
  if (cfg_k->rows == 0) return ok();
  Derived dk;
  (void)check_config(cfg_k, &dk);
  if ((st = check_planes(cfg_k, dk, k)) != KVQ_OK) return st;
  if (cfg_k->n_sink > 0 && !k->sink) return fail(KVQ_ERR_NULL, "sink plane is NULL");
  if (!q || !entropy || !workspace) return fail(KVQ_ERR_NULL, "q, entropy or workspace is NULL");
  if (!aligned16(q) || !aligned16(workspace) || (reinterpret_cast<uintptr_t>(entropy) & 3u))
    return fail(KVQ_ERR_ALIGN, "q and workspace must be 16-byte aligned, entropy 4-byte");
  if (lengths && (reinterpret_cast<uintptr_t>(lengths) & 3u)) return fail(KVQ_ERR_ALIGN, "lengths not 4-byte aligned");
  if (workspace_bytes < need) return fail(KVQ_ERR_SHAPE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  a.k_codes = static_cast<const uint8_t*>(k->codes);
  a.k_scale = static_cast<const uint16_t*>(k->scale);
  a.k_zero = static_cast<const uint16_t*>(k->zero);
  a.k_sink = static_cast<const uint16_t*>(k->sink);
  a.q = q;
  a.entropy = entropy;
  a.qrot = static_cast<float*>(workspace);
  a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    (size_t)(a.rows * q_heads * cfg_k->head_dim * 4 + 255) / 256 * 256);
  a.lengths = lengths;
  a.scale = scale;
  if ((a.rows * a.heads * a.n_chunks + 3) / 4 > 0x7fffffff || (a.rows * q_heads + 3) / 4 > 0x7fffffff)
    return fail(KVQ_ERR_SHAPE, "cache too large for one entropy launch");
  const int err = kvq::launch_entropy(a, stream);
  if (err != 0) return fail(KVQ_ERR_DEVICE, "attention entropy launch failed: %s", kvq::device_error_string(err));
  return ok();
}

kvq_status kvq_allocate_bits(const double* entropy, int64_t heads, int32_t total, int32_t lo, int32_t hi,
                             int32_t* bits) {
  if (!entropy || !bits) return fail(KVQ_ERR_NULL, "entropy or bits is NULL");
  if (heads <= 0 || heads > 32768) return fail(KVQ_ERR_SHAPE, "heads %lld (1 .. 32768)", (long long)heads);
  if (lo < 2 || hi > 4 || lo > hi) return fail(KVQ_ERR_BITS, "widths [%d, %d] (within 2 .. 4)", lo, hi);
  if ((int64_t)lo * heads > total || (int64_t)hi * heads < total)
    return fail(KVQ_ERR_PARAM, "total %d bits outside [%lld, %lld]", total, (long long)(lo * heads),
                (long long)(hi * heads));
  double sum = 0.0;
  for (int64_t i = 0; i < heads; ++i) {
    if (!(isfinite(entropy[i]) && entropy[i] >= 0.0)) return fail(KVQ_ERR_PARAM, "entropy[%lld] must be finite, >= 0", (long long)i);
    sum += entropy[i];
  }
  // the ideal share, floored into [lo, hi]; single bits by largest (smallest) remainder
  std::vector<double> x((size_t)heads);
  int64_t have = 0;
  for (int64_t i = 0; i < heads; ++i) {
    x[i] = sum > 0.0 ? (double)total * entropy[i] / sum : (double)total / (double)heads;
    const double f = floor(x[i]);
    bits[i] = (int32_t)(f < lo ? lo : (f > hi ? hi : f));
    have += bits[i];
  }
  while (have < total) {
    int64_t best = -1;
    for (int64_t i = 0; i < heads; ++i)
      if (bits[i] < hi && (best < 0 || x[i] - bits[i] > x[best] - bits[best])) best = i;
    ++bits[best];
    ++have;
  }
  while (have > total) {
    int64_t best = -1;
    for (int64_t i = 0; i < heads; ++i)
      if (bits[i] > lo && (best < 0 || x[i] - bits[i] <= x[best] - bits[best])) best = i;
    --bits[best];
    --have;
  }
  return ok();
}

kvq_status kvq_lloyd_max_gaussian(int32_t bits, double sigma, float* codebook_out) {
  if (!codebook_out) return fail(KVQ_ERR_NULL, "codebook_out is NULL");
  if (bits < 1 || bits > 5) return fail(KVQ_ERR_BITS, "bits %d (1..5)", bits);
  if (!(isfinite(sigma) && sigma > 0.0)) return fail(KVQ_ERR_PARAM, "sigma must be finite and > 0");
  const int n = 1 << bits;
  double c[32], lo[32], hi[32];
  // symmetric start, evenly spread over +-2 standard deviations
  for (int k = 0; k < n; ++k) c[k] = -2.0 + 4.0 * (k + 0.5) / n;
  for (int it = 0; it < 1000000; ++it) {
    for (int k = 0; k < n; ++k) {
      lo[k] = k == 0 ? -INFINITY : 0.5 * (c[k - 1] + c[k]);
      hi[k] = k == n - 1 ? INFINITY : 0.5 * (c[k] + c[k + 1]);
    }
    double moved = 0.0;
    for (int k = 0; k < n; ++k) {
      // mass of (a, b]; use the tail on the side that avoids cancellation
      double mass;
      if (lo[k] >= 0.0)
        mass = ntail(lo[k]) - ntail(hi[k]);
      else if (hi[k] <= 0.0)
        mass = ntail(-hi[k]) - ntail(-lo[k]);
      else
        mass = 1.0 - ntail(-lo[k]) - ntail(hi[k]);
      const double nc = (npdf(lo[k]) - npdf(hi[k])) / mass;
      moved = std::max(moved, fabs(nc - c[k]));
      c[k] = nc;
    }
    if (moved < 1e-14) break;
  }
  for (int k = 0; k < n; ++k) codebook_out[k] = (float)(c[k] * sigma);
  return ok();
}

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "required pointer is NULL";
    case KVQ_ERR_SHAPE: return "invalid shape or strides";
    case KVQ_ERR_BITS: return "unsupported bit width";
    case KVQ_ERR_GROUP: return "invalid group size";
    case KVQ_ERR_ROT: return "unknown enum value";
    case KVQ_ERR_PARAM: return "invalid parameter (perm, quaternion, codebook, rope, positions)";
    case KVQ_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_ABI: return "ABI version mismatch";
    case KVQ_ERR_DEVICE: return "HIP runtime error";
    case KVQ_ERR_INTERNAL: return "internal error";
  }
  return "unknown status";
}

const char* kvq_last_error_message(void) { return g_last_error.c_str(); }

}  // extern "C"

kvq_status kvq_rotor_matrix(const float* rq, int64_t head_dim, float tail_angle, float* out) {
  if (!rq || !out) return fail(KVQ_ERR_NULL, "rq or out is NULL");
  if (head_dim != 128 && head_dim != 256)
    return fail(KVQ_ERR_UNSUPPORTED, "head_dim %lld (supported: 128, 256)", (long long)head_dim);
  if (!isfinite(tail_angle)) return fail(KVQ_ERR_PARAM, "tail_angle must be finite");
  const int d = (int)head_dim, nb = d / 3;
  for (int b = 0; b < nb; ++b) {
    double n2 = 0.0;
    for (int k = 0; k < 4; ++k) {
      if (!isfinite(rq[4 * b + k])) return fail(KVQ_ERR_PARAM, "rq[%d] is not finite", b);
      n2 += (double)rq[4 * b + k] * rq[4 * b + k];
    }
    if (fabs(sqrt(n2) - 1.0) > 1e-4) return fail(KVQ_ERR_PARAM, "rq[%d] is not a unit quaternion", b);
  }
  memset(out, 0, sizeof(float) * (size_t)d * (size_t)d);
  for (int b = 0; b < nb; ++b) {
    // r (0, v) r* for r = (w, x, y, z): the homogeneous 3x3 form (equal to |r|^2 times the
    // rotation, so exact for the stored, nearly unit r)
    const double w = rq[4 * b], x = rq[4 * b + 1], y = rq[4 * b + 2], z = rq[4 * b + 3];
    const double m[3][3] = {{w * w + x * x - y * y - z * z, 2.0 * (x * y - w * z), 2.0 * (x * z + w * y)},
                            {2.0 * (x * y + w * z), w * w - x * x + y * y - z * z, 2.0 * (y * z - w * x)},
                            {2.0 * (x * z - w * y), 2.0 * (y * z + w * x), w * w - x * x - y * y + z * z}};
    for (int i = 0; i < 3; ++i)
      for (int j = 0; j < 3; ++j) out[(size_t)(3 * b + i) * d + 3 * b + j] = (float)m[i][j];
  }
  const int t0 = 3 * nb;
  if (d - t0 == 2) {
    const double c = cos((double)tail_angle), sn = sin((double)tail_angle);
    out[(size_t)t0 * d + t0] = (float)c;
    out[(size_t)t0 * d + t0 + 1] = (float)-sn;
    out[(size_t)(t0 + 1) * d + t0] = (float)sn;
    out[(size_t)(t0 + 1) * d + t0 + 1] = (float)c;
  } else if (d - t0 == 1) {
    out[(size_t)t0 * d + t0] = 1.0f;
  }
  return ok();
}
