// Kind-independent kernels: init, commit, error clear, streaming copy; and the
// dispatch of the kind-specific launchers.
#include "rssm_device.hpp"

namespace rssm {

__global__ __launch_bounds__(kThreads) void k_commit(Args a) {
  const Geom &g = a.g;
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= g.B * g.H) return;
  const int b = idx / g.H;
  const int64_t nc = a.n_committed[idx], nk = a.n_ckpt[idx];
  const int64_t hb = nc - nk;
  if (hb < 0 || hb > g.C) {
    atomicOr(a.err, RSSM_DEVERR_CURSOR);
    return;
  }
  const int acc = a.n_accept[b];
  if (acc < 0 || acc > a.T || hb + a.T > g.C) {
    atomicOr(a.err, RSSM_DEVERR_ACCEPT_RANGE);
    return;
  }
  a.n_committed[idx] = nc + acc;
}

// Commit for the snapshot path: cur[b] <- (cur[b] + n_accept[b]) mod S.
__global__ __launch_bounds__(kThreads) void k_commit_snapshot(Args a) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= a.g.B) return;
  const int S = a.snap_slots;
  const int cur = a.snap_cur[b];
  const int acc = a.n_accept[b];
  if (cur < 0 || cur >= S) {
    atomicOr(a.err, RSSM_DEVERR_CURSOR);
    return;
  }
  if (acc < 0 || acc > a.T) {
    atomicOr(a.err, RSSM_DEVERR_ACCEPT_RANGE);
    return;
  }
  a.snap_cur[b] = ring_add(cur, acc, S);
}

// Workgroups per sequence of the tree commit: each takes a range of key heads and the value
// heads that use them, about 8 KB of one record's rows, and at most 8 per sequence (Mamba-2
// B=512 64x128: 8; KDA 128x128: 4; GDN 128x128: 2).
__host__ __device__ inline int commit_tree_split(const Geom &g) {
  const int es = g.bf16 ? 2 : 4;
  const int64_t rec = (int64_t)g.H * (g.P + (g.kind == RSSM_KIND_KDA ? g.N : 1) + (g.kind != RSSM_KIND_MAMBA2 ? 1 : 0)) * es +
                      (int64_t)2 * g.G * g.N * es;
  int64_t s = rec / 8192;
  s = s < 1 ? 1 : (s > 8 ? 8 : s);
  return (int)(s < g.G ? s : g.G);
}

// Tree commit: the accepted path's records (every head's alpha, beta, v and every key
// head's k, q) move to the consecutive slots past the cursor, then every head's cursor
// replica advances.  Record i goes from offset path[i] to offset i; path[i] >= i, and a
// destination i is the source only of an entry j with path[j] = i, which needs j <= i.  So
// moving the records in path order reads every source before it is overwritten.
// A sequence is split over commit_tree_split(g) workgroups by key-head range (one per
// sequence left most of the GPU idle).  Each checks the path itself, reads the cursor
// replica of its first value head, moves its heads' rows and advances its heads' cursors,
// so no workgroup reads a cursor another one writes.
__global__ __launch_bounds__(kThreads) void k_commit_tree(Args a) {
  __shared__ int s_path[kMaxDrafts], s_par[kMaxDrafts];
  __shared__ int s_ok;
  const Geom &g = a.g;
  const int H = g.H, G = g.G, P = g.P, N = g.N, C = g.C;
  const int S = commit_tree_split(g), kpc = (G + S - 1) / S;
  const int b = blockIdx.x / S, chunk = blockIdx.x - b * S;
  const int g0 = chunk * kpc, g1 = g0 + kpc < G ? g0 + kpc : G;   // key heads [g0, g1)
  if (g0 >= g1) return;                                          // the same for the workgroup
  const int h0 = g0 * g.grp, h1 = g1 * g.grp;                    // their value heads
  const int t = threadIdx.x;
  const int T = a.T;
  const size_t BH = (size_t)g.B * H, BG = (size_t)g.B * G;   // rows per ring slot
  const int64_t nc = a.n_committed[(int64_t)b * H + h0], nk = a.n_ckpt[(int64_t)b * H + h0];
  const int64_t hb = nc - nk;
  if (hb < 0 || hb > C) {
    if (t == 0) atomicOr(a.err, RSSM_DEVERR_CURSOR);
    return;
  }
  const int acc = a.n_accept[b];
  if (t < T) {                               // the path and parent rows in one round trip
    s_path[t] = a.path[b * T + t];
    s_par[t] = a.parent[b * T + t];
  }
  __syncthreads();
  if (t == 0) {
    int ok = acc >= 0 && acc <= T && hb + T <= C;
    // the parent rows the verify accepted: each -1 or an earlier draft (otherwise the
    // verify appended nothing for this sequence)
    for (int d = 0; ok && d < T; ++d)
      if (s_par[d] < -1 || s_par[d] >= d) ok = 0;
    // a chain from the head; with valid parents every entry is a later draft than the
    // previous one, so path[i] >= i and the moves below read each source first
    int prev = -1;
    for (int j = 0; ok && j < acc; ++j) {
      const int d = s_path[j];
      if (d < 0 || d >= T || d <= prev || s_par[d] != prev)
        ok = 0;
      else
        prev = d;
    }
    s_ok = ok;
  }
  __syncthreads();
  if (!s_ok) {
    if (t == 0) atomicOr(a.err, RSSM_DEVERR_ACCEPT_RANGE);
    return;
  }
  // Each thread moves the same chunk positions of every record, so one thread's program
  // order already reads a chunk's source before any later record overwrites it.
  const int es = g.bf16 ? 2 : 4;
  const int slot0 = ring_mod(nc, C);
  const bool vec = (P * es) % 16 == 0;                        // rows in 16-byte chunks
  for (int i = 0; i < acc; ++i) {
    if (s_path[i] == i) continue;                            // already in place (uniform)
    const int src = ring_add(slot0, s_path[i], C), dst = ring_add(slot0, i, C);
    // scalar alpha (Mamba-2, GDN) and beta (GDN, KDA) of every value head
    const int f0 = g.kind == RSSM_KIND_KDA ? 1 : 0, f1 = g.kind == RSSM_KIND_MAMBA2 ? 1 : 2;
    for (int h = h0 + t; h < h1; h += kThreads) {
      const size_t hr = (size_t)b * H + h;
      for (int f = f0; f < f1; ++f) {
        const int64_t base = f == 0 ? g.off_alpha : g.off_beta;
        if (es == 2)
          *(uint16_t *)(a.ring + base + ((size_t)dst * BH + hr) * 2) = *(const uint16_t *)(a.ring + base + ((size_t)src * BH + hr) * 2);
        else
          *(uint32_t *)(a.ring + base + ((size_t)dst * BH + hr) * 4) = *(const uint32_t *)(a.ring + base + ((size_t)src * BH + hr) * 4);
      }
    }
    // k and q of the key heads: N * es is a multiple of 16 bytes for every dk
    const int ng = g1 - g0, cpk = N * es / 16, nk2 = 2 * ng * cpk;
    for (int c = t; c < nk2; c += kThreads) {
      const int row = c / cpk, part = c - row * cpk;          // cpk is a power of two
      const int which = row >= ng, gg = g0 + row - which * ng;
      const int64_t base = which ? g.off_q : g.off_k;
      const size_t kr = (size_t)b * G + gg;
      const uint8_t *ps = a.ring + base + ((size_t)src * BG + kr) * N * es + part * 16;
      uint8_t *pd = a.ring + base + ((size_t)dst * BG + kr) * N * es + part * 16;
      *(uint4 *)pd = *(const uint4 *)ps;
    }
    // KDA: the alpha row (dk elements, a whole number of 16-byte chunks) of the value heads
    if (g.kind == RSSM_KIND_KDA) {
      const int cpa = N * es / 16, na = (h1 - h0) * cpa;
      for (int c = t; c < na; c += kThreads) {
        const int h = h0 + c / cpa, part = c % cpa;
        const size_t hr = (size_t)b * H + h;
        const uint8_t *ps = a.ring + g.off_alpha + ((size_t)src * BH + hr) * N * es + part * 16;
        uint8_t *pd = a.ring + g.off_alpha + ((size_t)dst * BH + hr) * N * es + part * 16;
        *(uint4 *)pd = *(const uint4 *)ps;
      }
    }
    // v of the value heads
    if (vec) {
      const int cpv = P * es / 16, nvc = (h1 - h0) * cpv;
      for (int c = t; c < nvc; c += kThreads) {
        const int hl = g.cpv_lg >= 0 ? c >> g.cpv_lg : c / cpv, part = c - hl * cpv, h = h0 + hl;
        const size_t hr = (size_t)b * H + h;
        const uint8_t *ps = a.ring + g.off_v + ((size_t)src * BH + hr) * P * es + part * 16;
        uint8_t *pd = a.ring + g.off_v + ((size_t)dst * BH + hr) * P * es + part * 16;
        *(uint4 *)pd = *(const uint4 *)ps;
      }
    } else {
      for (int e = t; e < (h1 - h0) * P; e += kThreads) {
        const int h = h0 + e / P, pp = e % P;
        const size_t hr = (size_t)b * H + h;
        const size_t os = g.off_v + (((size_t)src * BH + hr) * P + pp) * es, od = g.off_v + (((size_t)dst * BH + hr) * P + pp) * es;
        if (es == 2)
          *(uint16_t *)(a.ring + od) = *(const uint16_t *)(a.ring + os);
        else
          *(uint32_t *)(a.ring + od) = *(const uint32_t *)(a.ring + os);
      }
    }
  }
  for (int h = h0 + t; h < h1; h += kThreads) a.n_committed[(int64_t)b * H + h] = nc + acc;
}

__global__ void k_clear_err(int32_t *err) {
  if (threadIdx.x == 0) *err = 0;
}

__global__ __launch_bounds__(kThreads) void k_stream_copy(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                         size_t n) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

hipError_t launch_init(const Args &a, hipStream_t s) {
  const dim3 grid((unsigned)(a.g.B * a.g.H));
#define CALL(n, r)                                                           \
  {                                                                          \
    hipLaunchKernelGGL((k_init<n, r>), grid, dim3(kThreads), 0, s, a);       \
    return hipGetLastError();                                                \
  }
  RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
#undef CALL
}

hipError_t launch_commit(const Args &a, hipStream_t s) {
  const int n = a.g.B * a.g.H;
  hipLaunchKernelGGL(k_commit, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_commit_tree(const Args &a, hipStream_t s) {
  hipLaunchKernelGGL(k_commit_tree, dim3((unsigned)(a.g.B * commit_tree_split(a.g))), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_commit_snapshot(const Args &a, hipStream_t s) {
  hipLaunchKernelGGL(k_commit_snapshot, dim3((unsigned)((a.g.B + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}


hipError_t launch_clear_err(int32_t *err, hipStream_t s) {
  hipLaunchKernelGGL(k_clear_err, dim3(1), dim3(64), 0, s, err);
  return hipGetLastError();
}

hipError_t launch_stream_copy(const void *src, void *dst, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  size_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 256 * 64) blocks = 256 * 64;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_stream_copy, dim3((unsigned)blocks), dim3(kThreads), 0, s, (const uint4 *)src, (uint4 *)dst, n);
  return hipGetLastError();
}

// Route a launch to the instances of the state's model kind and the call's staging path.
#define RSSM_ROUTE(FN)                                                   \
  {                                                                      \
    const int stg = stage_of(a);                                         \
    if (a.g.kind == RSSM_KIND_KDA) {                                     \
      if (stg == kStageBf16) return KindLaunch<RSSM_KIND_KDA, kStageBf16>::FN(a, s); \
      if (stg == kStageF32) return KindLaunch<RSSM_KIND_KDA, kStageF32>::FN(a, s);   \
      return KindLaunch<RSSM_KIND_KDA, kStageScalar>::FN(a, s);          \
    }                                                                    \
    if (a.g.kind == RSSM_KIND_GDN) {                                     \
      if (stg == kStageBf16) return KindLaunch<RSSM_KIND_GDN, kStageBf16>::FN(a, s); \
      if (stg == kStageF32) return KindLaunch<RSSM_KIND_GDN, kStageF32>::FN(a, s);   \
      return KindLaunch<RSSM_KIND_GDN, kStageScalar>::FN(a, s);          \
    }                                                                    \
    if (stg == kStageBf16) return KindLaunch<RSSM_KIND_MAMBA2, kStageBf16>::FN(a, s); \
    if (stg == kStageF32) return KindLaunch<RSSM_KIND_MAMBA2, kStageF32>::FN(a, s);   \
    return KindLaunch<RSSM_KIND_MAMBA2, kStageScalar>::FN(a, s);         \
  }

hipError_t launch_decode(const Args &a, hipStream_t s) RSSM_ROUTE(decode)
hipError_t launch_verify(const Args &a, hipStream_t s) RSSM_ROUTE(verify)
hipError_t launch_flush(const Args &a, hipStream_t s) RSSM_ROUTE(flush)
hipError_t launch_conventional(const Args &a, hipStream_t s) RSSM_ROUTE(conventional)
hipError_t launch_verify_snapshot(const Args &a, hipStream_t s) RSSM_ROUTE(verify_snapshot)
#undef RSSM_ROUTE

}  // namespace rssm
