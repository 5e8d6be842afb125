// Launchers of the decode, verify, flush, conventional and snapshot-verify kernels for one
// model kind and one record staging path.  Each kernels_<kind>_<path>.hip instantiates
// KindLaunch<KIND, STG> once, so the kernel instances spread over several translation units
// that compile in parallel.
#pragma once
#include "rssm_device.hpp"

namespace rssm {

namespace launch_detail {
inline dim3 grid_of(const Args &a) { return dim3((unsigned)(a.g.B * a.g.H)); }
}  // namespace launch_detail

template <int KIND, int STG>
hipError_t KindLaunch<KIND, STG>::decode(const Args &a, hipStream_t s) {
  using launch_detail::grid_of;
  const size_t lds = lds_bytes(KIND, a.g.C + 1, 1, a.g.P, a.g.N);
#define CALL(n, r)                                                                             \
  {                                                                                            \
    hipLaunchKernelGGL((k_decode<KIND, n, r, F, STG>), grid_of(a), dim3(kThreads), lds, s, a); \
    return hipGetLastError();                                                                  \
  }
  switch (a.g.read_copy) {
    case RSSM_READ_NONE: {
      constexpr int F = RSSM_READ_NONE;
      RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
    }
    case RSSM_READ_FP8: {
      constexpr int F = RSSM_READ_FP8;
      RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
    }
    case RSSM_READ_MXFP4: {
      constexpr int F = RSSM_READ_MXFP4;
      RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
    }
    default:
      return hipErrorInvalidValue;
  }
#undef CALL
}

// A fused fold (min_records > 0) writes the read copy in the state's format.
template <int KIND, int STG>
hipError_t KindLaunch<KIND, STG>::verify(const Args &a, hipStream_t s) {
  using launch_detail::grid_of;
  const size_t lds = lds_bytes(KIND, a.g.C, a.T, a.g.P, a.g.N);
#define CALL(n, r)                                                                                   \
  {                                                                                                  \
    hipLaunchKernelGGL((k_verify<KIND, n, r, FOLD, F, STG>), grid_of(a), dim3(kThreads), lds, s, a); \
    return hipGetLastError();                                                                        \
  }
  if (a.min_records <= 0) {
    constexpr bool FOLD = false;
    constexpr int F = RSSM_READ_NONE;
    RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
  }
  constexpr bool FOLD = true;
  switch (a.g.read_copy) {
    case RSSM_READ_NONE: {
      constexpr int F = RSSM_READ_NONE;
      RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
    }
    case RSSM_READ_FP8: {
      constexpr int F = RSSM_READ_FP8;
      RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
    }
    case RSSM_READ_MXFP4: {
      constexpr int F = RSSM_READ_MXFP4;
      RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
    }
    default:
      return hipErrorInvalidValue;
  }
#undef CALL
}

template <int KIND, int STG>
hipError_t KindLaunch<KIND, STG>::flush(const Args &a, hipStream_t s) {
  using launch_detail::grid_of;
  const size_t lds = lds_bytes(KIND, a.g.C, 1, a.g.P, a.g.N);
#define CALL(n, r)                                                                            \
  {                                                                                           \
    hipLaunchKernelGGL((k_flush<KIND, n, r, F, STG>), grid_of(a), dim3(kThreads), lds, s, a); \
    return hipGetLastError();                                                                 \
  }
  switch (a.g.read_copy) {
    case RSSM_READ_NONE: {
      constexpr int F = RSSM_READ_NONE;
      RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
    }
    case RSSM_READ_FP8: {
      constexpr int F = RSSM_READ_FP8;
      RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
    }
    case RSSM_READ_MXFP4: {
      constexpr int F = RSSM_READ_MXFP4;
      RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
    }
    default:
      return hipErrorInvalidValue;
  }
#undef CALL
}

template <int KIND, int STG>
hipError_t KindLaunch<KIND, STG>::conventional(const Args &a, hipStream_t s) {
  using launch_detail::grid_of;
  const size_t lds = lds_bytes(KIND, 1, 1, a.g.P, a.g.N);
#define CALL(n, r)                                                                              \
  {                                                                                             \
    hipLaunchKernelGGL((k_conventional<KIND, n, r, STG>), grid_of(a), dim3(kThreads), lds, s, a); \
    return hipGetLastError();                                                                   \
  }
  RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
#undef CALL
}

template <int KIND, int STG>
hipError_t KindLaunch<KIND, STG>::verify_snapshot(const Args &a, hipStream_t s) {
  using launch_detail::grid_of;
  const size_t lds = lds_bytes(KIND, a.T, a.T, a.g.P, a.g.N);
#define CALL(n, r)                                                                                 \
  {                                                                                                \
    hipLaunchKernelGGL((k_verify_snapshot<KIND, n, r, STG>), grid_of(a), dim3(kThreads), lds, s, a); \
    return hipGetLastError();                                                                      \
  }
  RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
#undef CALL
}

}  // namespace rssm
