// Internal definitions shared by the host layer (rssm_api.cpp) and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime.h>

#include "rssm.h"

namespace rssm {

constexpr int kThreads = 256;   // 4 waves of 64 per workgroup
constexpr int kWaves = 4;
constexpr int kMaxCapacity = 32;
constexpr int kMaxDrafts = 8;
constexpr int kMaxLdsBytes = 64 * 1024;
// Record staging paths (a kernel template parameter): 16-byte chunks of bf16 or fp32
// elements, or element-wise for layouts whose rows are not 16-byte aligned.
constexpr int kStageScalar = 0;
constexpr int kStageBf16 = 1;
constexpr int kStageF32 = 2;

// Everything a kernel needs to address one (sequence, value-head) tile.
struct Geom {
  int kind;        // RSSM_KIND_*
  int B, H, G, grp;
  int P, N;        // tile rows (dv) and columns (dk)
  int L, C;
  int bf16;        // inputs and ring are raw bf16 bits
  int cpv_lg;      // log2 of the 16-byte chunks per value row, -1 if not a power of two
  int read_copy;   // RSSM_READ_*
  int64_t off_alpha, off_beta, off_v, off_k, off_q;   // byte offsets inside the ring
};

struct Args {
  Geom g;
  float *s;                 // S_ckpt, or the conventional state
  uint8_t *s_read;
  uint8_t *s_read_scale;
  uint8_t *ring;
  int64_t *n_committed;
  int64_t *n_ckpt;
  int32_t *err;
  const void *alpha, *beta, *v, *k, *q;   // step or draft inputs
  float *out;                              // y [B][H][P] or O [B][T][H][P]
  const float *s0;                         // init source (may be null)
  const int32_t *n_accept;                 // commit
  const int32_t *parent;                   // tree verify / commit: [B][T] parent draft, -1 = head
  const int32_t *path;                     // tree commit: [B][T] accepted drafts in path order
  int T;                                   // drafts (verify / commit)
  int min_records;                         // flush threshold
  int vec16;                               // rows can be staged in 16-byte chunks
  int gather_out;                          // verify: output rows gathered in LDS, stored whole
  int32_t *snap_cur;                       // snapshot path: committed slot per sequence [B]
  int snap_slots;                          // snapshot path: slots per sequence (t_max + 1)
};

// Float offsets of the per-workgroup LDS arrays.  cap = records staged, T = queries.
// Rows of N floats (K, KDA's alpha) are padded by 4 floats.
struct LdsLayout {
  int alpha, beta, dec, coef, gam, misc, anc, q, r, K, V, o, total;
};

__host__ __device__ inline int up4(int x) { return (x + 3) & ~3; }

// out: T output rows of P floats at the end (verify with gathered output rows).
__host__ __device__ inline LdsLayout lds_layout(int kind, int cap, int T, int P, int N, bool out = false) {
  LdsLayout l;
  int o = 0;
  l.alpha = o; o += (kind == RSSM_KIND_KDA) ? cap * (N + 4) : up4(cap);   // KDA: an N-vector per record
  l.beta = o;  o += up4(cap);
  l.dec = o;   o += up4(T * cap);
  l.coef = o;  o += up4(T * cap);
  l.gam = o;   o += up4(T);
  l.misc = o;  o += 4;
  l.anc = o;   o += up4(2 * T);     // verify: draft parents and ancestor masks (int32)
  l.q = o;     o += T * N;
  l.r = o;     o += T * N;
  l.K = o;     o += cap * (N + 4);
  l.V = o;     o += up4(cap * P);
  l.o = o;     o += out ? up4(T * P) : 0;
  l.total = o;
  return l;
}

inline size_t lds_bytes(int kind, int cap, int T, int P, int N, bool out = false) {
  return (size_t)lds_layout(kind, cap, T, P, N, out).total * sizeof(float);
}

// Row groups of 8 handled per wave (the tile's P rows form ceil(P/8) groups over 4 waves),
// rounded up to a power of two.
inline int rgw_for(int P) {
  int rg = (P + 7) / 8;
  int per = (rg + kWaves - 1) / kWaves;
  int r = 1;
  while (r < per) r <<= 1;
  return r;
}

// Launchers (one per kernel family); return hipError_t.
hipError_t launch_decode(const Args &a, hipStream_t s);
hipError_t launch_verify(const Args &a, hipStream_t s);
hipError_t launch_flush(const Args &a, hipStream_t s);
hipError_t launch_conventional(const Args &a, hipStream_t s);
hipError_t launch_init(const Args &a, hipStream_t s);
hipError_t launch_commit(const Args &a, hipStream_t s);
hipError_t launch_commit_tree(const Args &a, hipStream_t s);
hipError_t launch_verify_snapshot(const Args &a, hipStream_t s);
hipError_t launch_commit_snapshot(const Args &a, hipStream_t s);
hipError_t launch_clear_err(int32_t *err, hipStream_t s);
hipError_t launch_stream_copy(const void *src, void *dst, size_t bytes, hipStream_t s);

// Launchers of one model kind and one staging path; each (kind, path) pair is instantiated
// in a source file of its own (kernels_<kind>_<path>.hip).
template <int KIND, int STG>
struct KindLaunch {
  static hipError_t decode(const Args &a, hipStream_t s);
  static hipError_t verify(const Args &a, hipStream_t s);
  static hipError_t flush(const Args &a, hipStream_t s);
  static hipError_t conventional(const Args &a, hipStream_t s);
  static hipError_t verify_snapshot(const Args &a, hipStream_t s);
};

inline int stage_of(const Args &a) { return !a.vec16 ? kStageScalar : (a.g.bf16 ? kStageBf16 : kStageF32); }

}  // namespace rssm
