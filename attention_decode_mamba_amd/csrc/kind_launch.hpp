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

// Mamba-2 decode with a read copy takes the one-wave-per-tile kernel where its layouts fit:
// 16-byte record chunks, N of 64 or 128, P <= 64 (at most 8 row groups in one wave) and a
// window of 2 to 16 records (so the ring has at least 2 slots and each slot's rows lie
// less than 4 GB apart).
template <int KIND, int STG>
hipError_t decode_rc(const Args &a, hipStream_t s, bool *taken) {
  *taken = false;
  if constexpr (KIND == RSSM_KIND_MAMBA2 && STG != kStageScalar) {
    const Geom &g = a.g;
    if (g.read_copy == RSSM_READ_NONE || (g.N != 64 && g.N != 128) || g.P > 64 || g.L < 2 || g.L > 16)
      return hipSuccess;
    *taken = true;
    const int groups = (g.B + kWaves - 1) / kWaves * g.H;
    const int wt = g.N == 64 ? WaveLds<64>::total : WaveLds<128>::total;
    const size_t lds = (size_t)(decode_rc_flag_offset(g.C + 1, g.P, g.N, wt) + kWaves) * sizeof(float);
    if (lds > (size_t)kMaxLdsBytes) {            // the flags past a fold layout at the budget's edge
      *taken = false;
      return hipSuccess;
    }
#define CALL(n, r)                                                                               \
  {                                                                                              \
    hipLaunchKernelGGL((k_decode_rc<n, r, F, STG>), dim3((unsigned)groups), dim3(kThreads), lds, s, a); \
    return hipGetLastError();                                                                    \
  }
#define RC_DISPATCH                                    \
  switch (g.N * 10 + rgw_for(g.P)) {                   \
    case 641: CALL(64, 1);                             \
    case 642: CALL(64, 2);                             \
    case 1281: CALL(128, 1);                           \
    case 1282: CALL(128, 2);                           \
    default: return hipErrorInvalidValue;              \
  }
    if (g.read_copy == RSSM_READ_FP8) {
      constexpr int F = RSSM_READ_FP8;
      RC_DISPATCH
    } else {
      constexpr int F = RSSM_READ_MXFP4;
      RC_DISPATCH
    }
#undef RC_DISPATCH
#undef CALL
  }
  return hipSuccess;
}

template <int KIND, int STG>
hipError_t KindLaunch<KIND, STG>::decode(const Args &a, hipStream_t s) {
  using launch_detail::grid_of;
  bool taken;
  const hipError_t e = decode_rc<KIND, STG>(a, s, &taken);
  if (taken) return e;
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
// The verify gathers its output rows in LDS when that still fits the LDS budget.
template <int KIND, int STG>
hipError_t KindLaunch<KIND, STG>::verify(const Args &a0, hipStream_t s) {
  using launch_detail::grid_of;
  Args a = a0;
  a.gather_out = lds_bytes(KIND, a.g.C, a.T, a.g.P, a.g.N, true) <= (size_t)kMaxLdsBytes;
  const size_t lds = lds_bytes(KIND, a.g.C, a.T, a.g.P, a.g.N, a.gather_out);
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
