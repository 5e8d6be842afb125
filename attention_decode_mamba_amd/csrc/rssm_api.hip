// Host layer of the C ABI (include/rssm.h): argument validation, buffer sizing,
// geometry setup and kernel launch.  Nothing is enqueued when validation fails.
#include <algorithm>
#include <string.h>

#include "rssm_internal.hpp"

using namespace rssm;

namespace {

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

bool dk_ok(int dk) { return dk == 32 || dk == 64 || dk == 128 || dk == 256; }

int check_cfg(const rssm_config *c) {
  if (!c) return RSSM_E_NULL;
  if (c->kind != RSSM_KIND_MAMBA2 && c->kind != RSSM_KIND_GDN && c->kind != RSSM_KIND_KDA) return RSSM_E_DTYPE;
  if (c->in_dtype != RSSM_DTYPE_F32 && c->in_dtype != RSSM_DTYPE_BF16) return RSSM_E_DTYPE;
  if (c->read_copy < RSSM_READ_NONE || c->read_copy > RSSM_READ_MXFP4) return RSSM_E_DTYPE;
  if (c->batch < 0 || c->n_heads < 1 || c->n_qk_heads < 1) return RSSM_E_SHAPE;
  if (c->n_heads % c->n_qk_heads) return RSSM_E_SHAPE;
  if (!dk_ok(c->dk)) return RSSM_E_SHAPE;
  if (c->dv < 1 || c->dv > 16384 / c->dk) return RSSM_E_SHAPE;
  if (c->L < 1 || c->t_max < 1 || c->t_max > kMaxDrafts) return RSSM_E_RANGE;
  if (c->capacity < c->L + c->t_max - 1 || c->capacity > kMaxCapacity) return RSSM_E_SHAPE;
  if ((int64_t)c->batch * c->n_heads > (int64_t)(1 << 30)) return RSSM_E_SHAPE;
  // ring and input element indices are computed in 32 bits on the device
  const int64_t lim = (int64_t)1 << 31;
  const int64_t rows_v = (int64_t)c->batch * c->n_heads, rows_k = (int64_t)c->batch * c->n_qk_heads;
  const int64_t slots = std::max<int64_t>(c->capacity, c->t_max);
  if (rows_v * slots * c->dv >= lim || rows_k * slots * c->dk >= lim) return RSSM_E_SHAPE;
  if (c->kind == RSSM_KIND_KDA && rows_v * slots * c->dk >= lim) return RSSM_E_SHAPE;
  if (lds_bytes(c->kind, c->capacity + 1, 1, c->dv, c->dk) > (size_t)kMaxLdsBytes) return RSSM_E_SHAPE;
  if (lds_bytes(c->kind, c->capacity, c->t_max, c->dv, c->dk) > (size_t)kMaxLdsBytes) return RSSM_E_SHAPE;
  return RSSM_OK;
}

void ring_layout(const rssm_config *c, int64_t off[5], int64_t *total) {
  const int64_t es = c->in_dtype == RSSM_DTYPE_BF16 ? 2 : 4;
  const int64_t B = c->batch, H = c->n_heads, G = c->n_qk_heads, C = c->capacity;
  const int64_t P = c->dv, N = c->dk;
  int64_t o = 0;
  off[0] = o;                                   // alpha [C][B][H] (KDA: [C][B][H][N])
  o = align256(o + B * H * C * (c->kind == RSSM_KIND_KDA ? N : 1) * es);
  off[1] = o;                                   // beta [C][B][H] (GDN and KDA)
  if (c->kind != RSSM_KIND_MAMBA2) o = align256(o + B * H * C * es);
  off[2] = o;                                   // v [C][B][H][P]
  o = align256(o + B * H * C * P * es);
  off[3] = o;                                   // k [C][B][G][N]
  o = align256(o + B * G * C * N * es);
  off[4] = o;                                   // q [C][B][G][N]
  o = align256(o + B * G * C * N * es);
  *total = o;
}

Geom make_geom(const rssm_config *c) {
  Geom g;
  g.kind = c->kind;
  g.B = c->batch;
  g.H = c->n_heads;
  g.G = c->n_qk_heads;
  g.grp = c->n_heads / c->n_qk_heads;
  g.P = c->dv;
  g.N = c->dk;
  g.L = c->L;
  g.C = c->capacity;
  g.bf16 = c->in_dtype == RSSM_DTYPE_BF16;
  {
    // log2 of the 16-byte chunks per value row (P * element size / 16), or -1 when that is
    // not a power of two (or not whole)
    const int bytes = c->dv * (g.bf16 ? 2 : 4);
    const int cpv = bytes / 16;
    g.cpv_lg = (bytes % 16 == 0 && cpv > 0 && (cpv & (cpv - 1)) == 0) ? __builtin_ctz(cpv) : -1;
  }
  g.read_copy = c->read_copy;
  int64_t off[5], total;
  ring_layout(c, off, &total);
  g.off_alpha = off[0];
  g.off_beta = off[1];
  g.off_v = off[2];
  g.off_k = off[3];
  g.off_q = off[4];
  return g;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int check_state(const rssm_config *c, const rssm_state *st, bool need_ring) {
  if (!st || !st->s_ckpt || !st->n_committed || !st->n_ckpt || !st->err) return RSSM_E_NULL;
  if (need_ring && !st->ring) return RSSM_E_NULL;
  if (c->read_copy != RSSM_READ_NONE && (!st->s_read || !st->s_read_scale)) return RSSM_E_NULL;
  if (!aligned(st->s_ckpt, 16) || !aligned(st->n_committed, 8) || !aligned(st->n_ckpt, 8) || !aligned(st->err, 4))
    return RSSM_E_ALIGN;
  if (c->read_copy != RSSM_READ_NONE && (!aligned(st->s_read, 16) || !aligned(st->s_read_scale, 4)))
    return RSSM_E_ALIGN;
  if (need_ring && !aligned(st->ring, 256)) return RSSM_E_ALIGN;
  return RSSM_OK;
}

int check_inputs(const rssm_config *c, const void *alpha, const void *beta, const void *v, const void *k,
                 const void *q, const float *out) {
  if (!alpha || !v || !k || !q || !out) return RSSM_E_NULL;
  if (c->kind != RSSM_KIND_MAMBA2 && !beta) return RSSM_E_NULL;
  const uintptr_t es = c->in_dtype == RSSM_DTYPE_BF16 ? 2 : 4;
  if (!aligned(alpha, es) || !aligned(v, es) || !aligned(k, es) || !aligned(q, es) || !aligned(out, 4))
    return RSSM_E_ALIGN;
  if (beta && !aligned(beta, es)) return RSSM_E_ALIGN;
  return RSSM_OK;
}

Args make_args(const rssm_config *c, const rssm_state *st) {
  Args a;
  memset(&a, 0, sizeof(a));
  a.g = make_geom(c);
  if (st) {
    a.s = st->s_ckpt;
    a.s_read = (uint8_t *)st->s_read;
    a.s_read_scale = (uint8_t *)st->s_read_scale;
    a.ring = (uint8_t *)st->ring;
    a.n_committed = st->n_committed;
    a.n_ckpt = st->n_ckpt;
    a.err = st->err;
  }
  return a;
}

int hip_status(hipError_t e) { return e == hipSuccess ? RSSM_OK : RSSM_E_HIP; }

// Rows can be moved in 16-byte chunks when a row is a whole number of chunks and every
// input row starts on a 16-byte boundary (ring rows then do too: the ring is 256-aligned).
// KDA's alpha rows (dk elements) are staged like key rows.
int vec16_ok(const rssm_config *c, const void *alpha, const void *v, const void *k, const void *q) {
  const int epc = c->in_dtype == RSSM_DTYPE_BF16 ? 8 : 4;
  if (c->dv % epc || c->dk % epc) return 0;
  if ((v && !aligned(v, 16)) || (k && !aligned(k, 16)) || (q && !aligned(q, 16))) return 0;
  if (c->kind == RSSM_KIND_KDA && alpha && !aligned(alpha, 16)) return 0;
  return 1;
}

}  // namespace

extern "C" {

int rssm_check_config(const rssm_config *cfg) { return check_cfg(cfg); }

int rssm_sizes(const rssm_config *cfg, rssm_buffer_sizes *out) {
  int r = check_cfg(cfg);
  if (r) return r;
  if (!out) return RSSM_E_NULL;
  const size_t tiles = (size_t)cfg->batch * cfg->n_heads;
  const size_t PN = (size_t)cfg->dv * cfg->dk;
  out->s_ckpt = tiles * PN * sizeof(float);
  out->s_read = cfg->read_copy == RSSM_READ_FP8 ? tiles * PN : cfg->read_copy == RSSM_READ_MXFP4 ? tiles * PN / 2 : 0;
  out->s_read_scale = cfg->read_copy == RSSM_READ_FP8     ? tiles * (PN / 32) * sizeof(float)
                      : cfg->read_copy == RSSM_READ_MXFP4 ? tiles * (PN / 32)
                                                          : 0;
  int64_t off[5], total;
  ring_layout(cfg, off, &total);
  out->ring = (size_t)total;
  out->n_committed = tiles * sizeof(int64_t);
  out->n_ckpt = tiles * sizeof(int64_t);
  out->err = sizeof(int32_t);
  return RSSM_OK;
}

int rssm_ring_offsets(const rssm_config *cfg, int64_t *out5) {
  int r = check_cfg(cfg);
  if (r) return r;
  if (!out5) return RSSM_E_NULL;
  int64_t total;
  ring_layout(cfg, out5, &total);
  return RSSM_OK;
}

int rssm_init_state(const rssm_config *cfg, const rssm_state *st, const float *s0, hipStream_t stream) {
  int r = check_cfg(cfg);
  if (r) return r;
  if ((r = check_state(cfg, st, false))) return r;
  if (s0 && !aligned(s0, 16)) return RSSM_E_ALIGN;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return RSSM_E_DEVICE;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return RSSM_E_DEVICE;
  if (cfg->batch == 0) return hip_status(launch_clear_err(st->err, stream));
  Args a = make_args(cfg, st);
  a.s0 = s0;
  return hip_status(launch_init(a, stream));
}

int rssm_decode_step(const rssm_config *cfg, const rssm_state *st, const void *alpha, const void *beta,
                     const void *v, const void *k, const void *q, float *y, hipStream_t stream) {
  int r = check_cfg(cfg);
  if (r) return r;
  if ((r = check_state(cfg, st, true))) return r;
  if ((r = check_inputs(cfg, alpha, beta, v, k, q, y))) return r;
  if (cfg->batch == 0) return RSSM_OK;
  Args a = make_args(cfg, st);
  a.alpha = alpha;
  a.beta = beta;
  a.v = v;
  a.k = k;
  a.q = q;
  a.out = y;
  a.vec16 = vec16_ok(cfg, alpha, v, k, q);
  return hip_status(launch_decode(a, stream));
}

int rssm_flush(const rssm_config *cfg, const rssm_state *st, int32_t min_records, hipStream_t stream) {
  int r = check_cfg(cfg);
  if (r) return r;
  if ((r = check_state(cfg, st, true))) return r;
  if (min_records < 0) return RSSM_E_RANGE;
  if (cfg->batch == 0) return RSSM_OK;
  Args a = make_args(cfg, st);
  a.min_records = min_records;
  a.vec16 = vec16_ok(cfg, nullptr, nullptr, nullptr, nullptr);
  return hip_status(launch_flush(a, stream));
}

int rssm_verify(const rssm_config *cfg, const rssm_state *st, int32_t T, const void *alpha, const void *beta,
                const void *v, const void *k, const void *q, float *o, hipStream_t stream) {
  int r = check_cfg(cfg);
  if (r) return r;
  if ((r = check_state(cfg, st, true))) return r;
  if (T < 1 || T > cfg->t_max) return RSSM_E_RANGE;
  if ((r = check_inputs(cfg, alpha, beta, v, k, q, o))) return r;
  if (cfg->batch == 0) return RSSM_OK;
  Args a = make_args(cfg, st);
  a.alpha = alpha;
  a.beta = beta;
  a.v = v;
  a.k = k;
  a.q = q;
  a.out = o;
  a.T = T;
  a.vec16 = vec16_ok(cfg, alpha, v, k, q);
  return hip_status(launch_verify(a, stream));
}

int rssm_commit(const rssm_config *cfg, const rssm_state *st, const int32_t *n_accept, int32_t T,
                hipStream_t stream) {
  int r = check_cfg(cfg);
  if (r) return r;
  if ((r = check_state(cfg, st, false))) return r;
  if (!n_accept) return RSSM_E_NULL;
  if (!aligned(n_accept, 4)) return RSSM_E_ALIGN;
  if (T < 1 || T > cfg->t_max) return RSSM_E_RANGE;
  if (cfg->batch == 0) return RSSM_OK;
  Args a = make_args(cfg, st);
  a.n_accept = n_accept;
  a.T = T;
  return hip_status(launch_commit(a, stream));
}

int rssm_verify_tree(const rssm_config *cfg, const rssm_state *st, int32_t T, const int32_t *parent,
                     const void *alpha, const void *beta, const void *v, const void *k, const void *q, float *o,
                     hipStream_t stream) {
  int r = check_cfg(cfg);
  if (r) return r;
  if ((r = check_state(cfg, st, true))) return r;
  if (T < 1 || T > cfg->t_max) return RSSM_E_RANGE;
  if (!parent) return RSSM_E_NULL;
  if (!aligned(parent, 4)) return RSSM_E_ALIGN;
  if ((r = check_inputs(cfg, alpha, beta, v, k, q, o))) return r;
  if (cfg->batch == 0) return RSSM_OK;
  Args a = make_args(cfg, st);
  a.alpha = alpha;
  a.beta = beta;
  a.v = v;
  a.k = k;
  a.q = q;
  a.out = o;
  a.T = T;
  a.parent = parent;
  a.vec16 = vec16_ok(cfg, alpha, v, k, q);
  return hip_status(launch_verify(a, stream));
}

int rssm_verify_fold(const rssm_config *cfg, const rssm_state *st, int32_t min_records, int32_t T,
                     const int32_t *parent, const void *alpha, const void *beta, const void *v, const void *k,
                     const void *q, float *o, hipStream_t stream) {
  int r = check_cfg(cfg);
  if (r) return r;
  if ((r = check_state(cfg, st, true))) return r;
  if (min_records < 0) return RSSM_E_RANGE;
  if (T < 1 || T > cfg->t_max) return RSSM_E_RANGE;
  if (parent && !aligned(parent, 4)) return RSSM_E_ALIGN;
  if ((r = check_inputs(cfg, alpha, beta, v, k, q, o))) return r;
  if (cfg->batch == 0) return RSSM_OK;
  Args a = make_args(cfg, st);
  a.alpha = alpha;
  a.beta = beta;
  a.v = v;
  a.k = k;
  a.q = q;
  a.out = o;
  a.T = T;
  a.parent = parent;
  a.min_records = min_records > 1 ? min_records : 1;  // the fold threshold of rssm_flush
  a.vec16 = vec16_ok(cfg, alpha, v, k, q);
  return hip_status(launch_verify(a, stream));
}

int rssm_commit_tree(const rssm_config *cfg, const rssm_state *st, const int32_t *parent, const int32_t *path,
                     const int32_t *n_accept, int32_t T, hipStream_t stream) {
  int r = check_cfg(cfg);
  if (r) return r;
  if ((r = check_state(cfg, st, true))) return r;
  if (!parent || !path || !n_accept) return RSSM_E_NULL;
  if (!aligned(parent, 4) || !aligned(path, 4) || !aligned(n_accept, 4)) return RSSM_E_ALIGN;
  if (T < 1 || T > cfg->t_max) return RSSM_E_RANGE;
  if (cfg->batch == 0) return RSSM_OK;
  Args a = make_args(cfg, st);
  a.parent = parent;
  a.path = path;
  a.n_accept = n_accept;
  a.T = T;
  return hip_status(launch_commit_tree(a, stream));
}

int rssm_verify_snapshot(const rssm_config *cfg, float *snap, const int32_t *cur, int32_t T, const void *alpha,
                         const void *beta, const void *v, const void *k, const void *q, float *o, int32_t *err,
                         hipStream_t stream) {
  int r = check_cfg(cfg);
  if (r) return r;
  if (!snap || !cur || !err) return RSSM_E_NULL;
  if (!aligned(snap, 16) || !aligned(cur, 4) || !aligned(err, 4)) return RSSM_E_ALIGN;
  if (T < 1 || T > cfg->t_max) return RSSM_E_RANGE;
  if ((r = check_inputs(cfg, alpha, beta, v, k, q, o))) return r;
  if (cfg->batch == 0) return RSSM_OK;
  Args a = make_args(cfg, nullptr);
  a.s = snap;
  a.snap_cur = const_cast<int32_t *>(cur);
  a.snap_slots = cfg->t_max + 1;
  a.err = err;
  a.alpha = alpha;
  a.beta = beta;
  a.v = v;
  a.k = k;
  a.q = q;
  a.out = o;
  a.T = T;
  a.vec16 = vec16_ok(cfg, alpha, v, k, q);
  return hip_status(launch_verify_snapshot(a, stream));
}

int rssm_commit_snapshot(const rssm_config *cfg, int32_t *cur, const int32_t *n_accept, int32_t T, int32_t *err,
                         hipStream_t stream) {
  int r = check_cfg(cfg);
  if (r) return r;
  if (!cur || !n_accept || !err) return RSSM_E_NULL;
  if (!aligned(cur, 4) || !aligned(n_accept, 4) || !aligned(err, 4)) return RSSM_E_ALIGN;
  if (T < 1 || T > cfg->t_max) return RSSM_E_RANGE;
  if (cfg->batch == 0) return RSSM_OK;
  Args a = make_args(cfg, nullptr);
  a.snap_cur = cur;
  a.snap_slots = cfg->t_max + 1;
  a.err = err;
  a.n_accept = n_accept;
  a.T = T;
  return hip_status(launch_commit_snapshot(a, stream));
}

int rssm_decode_step_conventional(const rssm_config *cfg, float *s, const void *alpha, const void *beta,
                                  const void *v, const void *k, const void *q, float *y, hipStream_t stream) {
  int r = check_cfg(cfg);
  if (r) return r;
  if (!s) return RSSM_E_NULL;
  if (!aligned(s, 16)) return RSSM_E_ALIGN;
  if ((r = check_inputs(cfg, alpha, beta, v, k, q, y))) return r;
  if (cfg->batch == 0) return RSSM_OK;
  Args a = make_args(cfg, nullptr);
  a.s = s;
  a.alpha = alpha;
  a.beta = beta;
  a.v = v;
  a.k = k;
  a.q = q;
  a.out = y;
  a.vec16 = vec16_ok(cfg, alpha, v, k, q);
  return hip_status(launch_conventional(a, stream));
}

int rssm_get_error(const rssm_state *st, hipStream_t stream) {
  if (!st || !st->err) return RSSM_E_NULL;
  if (hipStreamSynchronize(stream) != hipSuccess) return RSSM_E_HIP;
  int32_t h = 0;
  if (hipMemcpy(&h, st->err, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return RSSM_E_HIP;
  if (launch_clear_err(st->err, stream) != hipSuccess) return RSSM_E_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return RSSM_E_HIP;
  return h;
}

int rssm_stream_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
  if (!src || !dst) return RSSM_E_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16) || bytes % 16) return RSSM_E_ALIGN;
  return hip_status(launch_stream_copy(src, dst, bytes, stream));
}

const char *rssm_strerror(int code) {
  switch (code) {
    case RSSM_OK: return "ok";
    case RSSM_E_NULL: return "a required pointer is NULL";
    case RSSM_E_SHAPE: return "unsupported or inconsistent sizes";
    case RSSM_E_DTYPE: return "unknown kind, input dtype or read-copy format";
    case RSSM_E_ALIGN: return "misaligned pointer or size";
    case RSSM_E_RANGE: return "argument out of range";
    case RSSM_E_HIP: return "HIP runtime call failed";
    case RSSM_E_DEVICE: return "no usable gfx950 device";
    default: break;
  }
  if (code > 0) {
    if (code & RSSM_DEVERR_CURSOR) return "device: inconsistent cursor counters";
    if (code & RSSM_DEVERR_VERIFY_CAPACITY) return "device: verify would overflow the ring (h + T > capacity)";
    if (code & RSSM_DEVERR_ACCEPT_RANGE) return "device: accepted count out of range";
    if (code & RSSM_DEVERR_TREE) return "device: draft tree with a parent that is not -1 or an earlier draft";
  }
  return "unknown error";
}

int rssm_version(void) { return 100; }

}  // extern "C"
