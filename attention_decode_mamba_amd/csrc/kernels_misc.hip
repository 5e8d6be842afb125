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
