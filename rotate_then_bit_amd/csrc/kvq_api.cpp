// Host side of the kvq C ABI: argument checking, plane sizes, kernel-argument
// marshalling and dispatch.  Every check runs before anything is enqueued, so
// an error return means no work was done.  No HIP call is made on an error path.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

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
};

kvq_status check_config(const kvq_config* cfg, Derived* dv) {
  if (!cfg) return fail(KVQ_ERR_NULL, "cfg is NULL");
  if (cfg->abi_version != KVQ_ABI_VERSION)
    return fail(KVQ_ERR_ABI, "abi_version %d, library is %d", cfg->abi_version, KVQ_ABI_VERSION);
  if (cfg->dtype < KVQ_F16 || cfg->dtype > KVQ_F32) return fail(KVQ_ERR_ROT, "unknown dtype %d", cfg->dtype);
  if (cfg->rot < KVQ_ROT_NONE || cfg->rot > KVQ_ROT_SO4) return fail(KVQ_ERR_ROT, "unknown rotation %d", cfg->rot);
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
  if (cfg->pos_offset < 0 || cfg->pos_offset + cfg->tokens > (int64_t(1) << 31))
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
  if (cfg->quant == KVQ_Q_LLOYD) {
    if (!cfg->codebook) return fail(KVQ_ERR_NULL, "codebook is required for Lloyd-Max");
    const int n_levels = 1 << cfg->bits;
    for (int i = 0; i < n_levels; ++i) {
      if (!isfinite(cfg->codebook[i])) return fail(KVQ_ERR_PARAM, "codebook entry %d not finite", i);
      if (i > 0 && !(cfg->codebook[i] > cfg->codebook[i - 1]))
        return fail(KVQ_ERR_PARAM, "codebook not strictly ascending at %d", i);
    }
  }
  dv->n_vec = rth;
  dv->code_bytes = d * cfg->bits / 8;
  dv->ngroups = cfg->quant == KVQ_Q_MINMAX ? d / cfg->group_size : 0;
  return KVQ_OK;
}

void plane_sizes(const kvq_config* cfg, const Derived& dv, size_t* codes, size_t* scale, size_t* zero,
                 size_t* norm, size_t* sink) {
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
  if (cfg->quant == KVQ_Q_LLOYD) memcpy(a->codebook, cfg->codebook, sizeof(float) * (1 << cfg->bits));
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
                            size_t* sink) {
  Derived dv;
  kvq_status st = check_config(cfg, &dv);
  if (st != KVQ_OK) return st;
  if (!codes || !scale || !zero || !norm || !sink) return fail(KVQ_ERR_NULL, "size output pointer is NULL");
  plane_sizes(cfg, dv, codes, scale, zero, norm, sink);
  return ok();
}

kvq_status kvq_encode(const kvq_config* cfg, const void* x, const kvq_planes* out, void* stream) {
  Derived dv;
  kvq_status st = check_config(cfg, &dv);
  if (st != KVQ_OK) return st;
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
  plan_work(cfg, &a);
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
  if (err != 0) return fail(KVQ_ERR_DEVICE, "encode launch failed: %s", kvq::device_error_string(err));
  return ok();
}

kvq_status kvq_append(const kvq_config* cfg, const void* x, const int64_t* positions, const kvq_planes* cache,
                      void* stream) {
  Derived dv;
  kvq_status st = check_config(cfg, &dv);  // cfg describes the cache: tokens = slots per row
  if (st != KVQ_OK) return st;
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
  plan_work(cfg, &a);
  const bool d128 = cfg->head_dim == 128;
  int err;
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
  if (err != 0) return fail(KVQ_ERR_DEVICE, "decode launch failed: %s", kvq::device_error_string(err));
  return ok();
}

namespace {
// the configurations decode-step attention supports, and the workspace it needs
kvq_status check_attend(const kvq_config* cfg_k, const kvq_config* cfg_v, int64_t q_heads, size_t* ws_bytes,
                        kvq::AttendArgs* a) {
  Derived dk, dv;
  kvq_status st = check_config(cfg_k, &dk);
  if (st != KVQ_OK) return st;
  if (cfg_v) {
    if ((st = check_config(cfg_v, &dv)) != KVQ_OK) return st;
    if (cfg_v->rows != cfg_k->rows || cfg_v->tokens != cfg_k->tokens || cfg_v->heads != cfg_k->heads ||
        cfg_v->head_dim != cfg_k->head_dim || cfg_v->bits != cfg_k->bits || cfg_v->group_size != cfg_k->group_size ||
        cfg_v->n_sink != cfg_k->n_sink || cfg_v->pos_offset != cfg_k->pos_offset || cfg_v->rot != cfg_k->rot ||
        cfg_v->quant != cfg_k->quant)
      return fail(KVQ_ERR_SHAPE, "the K and V caches must share rows, slots, heads, head_dim, bits, group, "
                                 "sinks, pos_offset, rotation and quantizer");
  }
  if (cfg_k->head_dim != 128 || cfg_k->rot != KVQ_ROT_FWHT || cfg_k->quant != KVQ_Q_MINMAX ||
      (cfg_k->bits != 2 && cfg_k->bits != 4) || cfg_k->group_size < 32 || cfg_k->group_size > 128)
    return fail(KVQ_ERR_UNSUPPORTED, "attention supports head_dim 128, Walsh-Hadamard, min-max, 2 or 4 bits, "
                                     "groups of 32, 64 or 128");
  if (cfg_k->pos_offset != 0) return fail(KVQ_ERR_UNSUPPORTED, "attention needs pos_offset 0 (slot = position)");
  if (cfg_k->n_sink > 64) return fail(KVQ_ERR_UNSUPPORTED, "attention supports at most 64 sink slots");
  if (cfg_k->heads <= 0 || q_heads <= 0 || q_heads % cfg_k->heads != 0)
    return fail(KVQ_ERR_SHAPE, "q_heads must be a positive multiple of heads");
  const int64_t qg = q_heads / cfg_k->heads;
  if (qg != 1 && qg != 2 && qg != 4)
    return fail(KVQ_ERR_UNSUPPORTED, "attention supports 1, 2 or 4 query heads per KV head");
  int32_t nc = 1, ct = 8;
  const bool mma_blk = cfg_k->group_size == 128 && cfg_k->heads % 4 == 0;  // bits are 2 or 4 here
  kvq::attend_chunks(cfg_k->rows, cfg_k->heads, cfg_k->tokens, mma_blk, &nc, &ct);
  int64_t nq = 0, tmp = 0;
  if (!mul_ok(cfg_k->rows, q_heads, &nq) || !mul_ok(nq, (int64_t)nc * kvq::kAttendPart + 128, &tmp) ||
      tmp > (int64_t(1) << 40))
    return fail(KVQ_ERR_SHAPE, "attention workspace too large");
  const size_t q_bytes = (size_t)(nq * 128 * 4 + 255) / 256 * 256;
  *ws_bytes = q_bytes + (size_t)nq * (size_t)nc * kvq::kAttendPart * 4;
  if (a) {
    memset(a, 0, sizeof *a);
    a->rows = cfg_k->rows;
    a->tokens = cfg_k->tokens;
    a->heads = cfg_k->heads;
    a->q_heads = q_heads;
    a->group_log2 = ilog2(cfg_k->group_size);
    a->n_sink = cfg_k->n_sink;
    a->n_chunks = nc;
    a->chunk = ct;
    a->use_perm_k = cfg_k->perm ? 1 : 0;
    if (cfg_k->perm)
      for (int i = 0; i < 128; ++i) a->perm_k[i] = (uint8_t)cfg_k->perm[i];
    if (cfg_v) {
      a->use_perm_v = cfg_v->perm ? 1 : 0;
      if (cfg_v->perm)
        for (int i = 0; i < 128; ++i) a->perm_v[i] = (uint8_t)cfg_v->perm[i];
    }
  }
  return KVQ_OK;
}
}  // namespace

kvq_status kvq_attend_workspace_size(const kvq_config* cfg_k, int64_t q_heads, size_t* bytes) {
  if (!bytes) return fail(KVQ_ERR_NULL, "bytes is NULL");
  kvq_status st = check_attend(cfg_k, nullptr, q_heads, bytes, nullptr);
  return st == KVQ_OK ? ok() : st;
}

kvq_status kvq_attend(const kvq_config* cfg_k, const kvq_planes* k, const kvq_config* cfg_v, const kvq_planes* v,
                      const float* q, int64_t q_heads, const int32_t* lengths, float scale, float* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!cfg_v) return fail(KVQ_ERR_NULL, "cfg_v is NULL");
  size_t need = 0;
  kvq::AttendArgs a;
  kvq_status st = check_attend(cfg_k, cfg_v, q_heads, &need, &a);
  if (st != KVQ_OK) return st;
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return fail(KVQ_ERR_PARAM, "scale must be finite");
  Derived dk, dv;
  (void)check_config(cfg_k, &dk);  // both already accepted above; this fills the derived sizes
  (void)check_config(cfg_v, &dv);
  if (!k || !v) return fail(KVQ_ERR_NULL, "planes is NULL");
  if (cfg_k->rows == 0) return ok();
  // (a cache with no slot still runs: every output row is then zero)
  if ((st = check_planes(cfg_k, dk, k)) != KVQ_OK) return st;
  if ((st = check_planes(cfg_v, dv, v)) != KVQ_OK) return st;
  if (cfg_k->n_sink > 0 && (!k->sink || !v->sink)) return fail(KVQ_ERR_NULL, "sink plane is NULL");
  if (!q || !out || !workspace) return fail(KVQ_ERR_NULL, "q, out or workspace is NULL");
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace))
    return fail(KVQ_ERR_ALIGN, "q, out and workspace must be 16-byte aligned");
  if (lengths && (reinterpret_cast<uintptr_t>(lengths) & 3u)) return fail(KVQ_ERR_ALIGN, "lengths not 4-byte aligned");
  if (workspace_bytes < need)
    return fail(KVQ_ERR_SHAPE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
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
  a.qrot = static_cast<float*>(workspace);
  a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + (size_t)(a.rows * q_heads * 128 * 4 + 255) / 256 * 256);
  a.lengths = lengths;
  a.scale = scale;
  const int err = kvq::launch_attend(cfg_k->bits, (int)(q_heads / cfg_k->heads), a, stream);
  if (err != 0) return fail(KVQ_ERR_DEVICE, "attention launch failed: %s", kvq::device_error_string(err));
  return ok();
}

kvq_status kvq_lloyd_max_gaussian(int32_t bits, double sigma, float* codebook_out) {
  if (!codebook_out) return fail(KVQ_ERR_NULL, "codebook_out is NULL");
  if (bits < 1 || bits > 4) return fail(KVQ_ERR_BITS, "bits %d (1..4)", bits);
  if (!(isfinite(sigma) && sigma > 0.0)) return fail(KVQ_ERR_PARAM, "sigma must be finite and > 0");
  const int n = 1 << bits;
  double c[16], lo[16], hi[16];
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
