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

// Tree commit: the accepted path's records move to the consecutive slots past the cursor,
// then the cursor advances.  Two phases through LDS: every source is read before any
// destination is written (a destination can be the source of a later path entry).  One
// workgroup per (sequence, value head); the first value head of a key group moves k and q.
__global__ __launch_bounds__(kThreads) void k_commit_tree(Args a) {
  extern __shared__ uint32_t buf[];
  __shared__ int s_path[kMaxDrafts];
  __shared__ int s_ok;
  const Geom &g = a.g;
  const int tile = blockIdx.x;
  const int b = tile / g.H, hh = tile - b * g.H, gq = hh / g.grp;
  const bool lead = (hh % g.grp) == 0;
  const int t = threadIdx.x;
  const int T = a.T;
  const int64_t nc = a.n_committed[tile], nk = a.n_ckpt[tile];
  const int64_t hb = nc - nk;
  if (hb < 0 || hb > g.C) {
    if (t == 0) atomicOr(a.err, RSSM_DEVERR_CURSOR);
    return;
  }
  const int acc = a.n_accept[b];
  if (t == 0) {
    int ok = acc >= 0 && acc <= T && hb + T <= g.C;
    int prev = -1;
    for (int j = 0; ok && j < acc; ++j) {
      const int d = a.path[b * T + j];
      if (d < 0 || d >= T || a.parent[b * T + d] != prev) {
        ok = 0;
      } else {
        s_path[j] = d;
        prev = d;
      }
    }
    s_ok = ok;
  }
  __syncthreads();
  if (!s_ok) {
    if (t == 0) atomicOr(a.err, RSSM_DEVERR_ACCEPT_RANGE);
    return;
  }
  const int P = g.P, N = g.N, C = g.C;
  const int es = g.bf16 ? 2 : 4;
  const int nsc = g.kind == RSSM_KIND_GDN ? 2 : 1;          // alpha (and beta)
  const int per = nsc + P + (lead ? 2 * N : 0);
  const int total = acc * per;
  const int slot0 = ring_mod(nc, C);
  // element e of the record in ring slot `slot`
  auto addr = [&](int e, int slot) -> uint8_t * {
    const int hr = (b * g.H + hh) * C + slot;
    const int kr = (b * g.G + gq) * C + slot;
    if (e == 0) return a.ring + g.off_alpha + (size_t)hr * es;
    if (e < nsc) return a.ring + g.off_beta + (size_t)hr * es;
    e -= nsc;
    if (e < P) return a.ring + g.off_v + ((size_t)hr * P + e) * es;
    e -= P;
    if (e < N) return a.ring + g.off_k + ((size_t)kr * N + e) * es;
    return a.ring + g.off_q + ((size_t)kr * N + e - N) * es;
  };
  for (int i = t; i < total; i += kThreads) {
    const int j = i / per, e = i - j * per;
    if (s_path[j] == j) continue;                          // already in place
    const uint8_t *src = addr(e, ring_add(slot0, s_path[j], C));
    buf[i] = es == 2 ? (uint32_t) * (const uint16_t *)src : *(const uint32_t *)src;
  }
  __syncthreads();
  for (int i = t; i < total; i += kThreads) {
    const int j = i / per, e = i - j * per;
    if (s_path[j] == j) continue;
    uint8_t *dst = addr(e, ring_add(slot0, j, C));
    if (es == 2)
      *(uint16_t *)dst = (uint16_t)buf[i];
    else
      *(uint32_t *)dst = buf[i];
  }
  if (t == 0) a.n_committed[tile] = nc + acc;
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
  const size_t lds = (size_t)a.T * (2 + a.g.P + 2 * a.g.N) * sizeof(uint32_t);
  hipLaunchKernelGGL(k_commit_tree, dim3((unsigned)(a.g.B * a.g.H)), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_commit_snapshot(const Args &a, hipStream_t s) {
  hipLaunchKernelGGL(k_commit_snapshot, dim3((unsigned)((a.g.B + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_verify_snapshot(const Args &a, hipStream_t s) {
  return a.g.kind == RSSM_KIND_GDN ? launch_verify_snapshot_gdn(a, s) : launch_verify_snapshot_m2(a, s);
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

hipError_t launch_decode(const Args &a, hipStream_t s) {
  return a.g.kind == RSSM_KIND_GDN ? launch_decode_gdn(a, s) : launch_decode_m2(a, s);
}
hipError_t launch_verify(const Args &a, hipStream_t s) {
  return a.g.kind == RSSM_KIND_GDN ? launch_verify_gdn(a, s) : launch_verify_m2(a, s);
}
hipError_t launch_flush(const Args &a, hipStream_t s) {
  return a.g.kind == RSSM_KIND_GDN ? launch_flush_gdn(a, s) : launch_flush_m2(a, s);
}
hipError_t launch_conventional(const Args &a, hipStream_t s) {
  return a.g.kind == RSSM_KIND_GDN ? launch_conventional_gdn(a, s) : launch_conventional_m2(a, s);
}

}  // namespace rssm
