// Gated DeltaNet instances of the decode, verify, flush and conventional kernels.
#include "rssm_device.hpp"

namespace rssm {

namespace {
constexpr int kKind = RSSM_KIND_GDN;

inline dim3 grid_of(const Args &a) { return dim3((unsigned)(a.g.B * a.g.H)); }
}  // namespace

hipError_t launch_decode_gdn(const Args &a, hipStream_t s) {
  const size_t lds = lds_bytes(kKind, a.g.C + 1, 1, a.g.P, a.g.N);
#define CALL(n, r)                                                                             \
  {                                                                                            \
    hipLaunchKernelGGL((k_decode<kKind, n, r, F>), grid_of(a), dim3(kThreads), lds, s, a);     \
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

hipError_t launch_verify_gdn(const Args &a, hipStream_t s) {
  const size_t lds = lds_bytes(kKind, a.g.C, a.T, a.g.P, a.g.N);
  // a fused fold (min_records > 0) writes the read copy in the state's format
  const int variant = a.min_records > 0 ? 1 + a.g.read_copy : 0;
#define CALL(n, r)                                                                                 \
  {                                                                                                \
    switch (variant) {                                                                             \
      case 0: hipLaunchKernelGGL((k_verify<kKind, n, r, false, RSSM_READ_NONE>), grid_of(a), dim3(kThreads), lds, s, a); break; \
      case 1 + RSSM_READ_NONE: hipLaunchKernelGGL((k_verify<kKind, n, r, true, RSSM_READ_NONE>), grid_of(a), dim3(kThreads), lds, s, a); break; \
      case 1 + RSSM_READ_FP8: hipLaunchKernelGGL((k_verify<kKind, n, r, true, RSSM_READ_FP8>), grid_of(a), dim3(kThreads), lds, s, a); break; \
      case 1 + RSSM_READ_MXFP4: hipLaunchKernelGGL((k_verify<kKind, n, r, true, RSSM_READ_MXFP4>), grid_of(a), dim3(kThreads), lds, s, a); break; \
      default: return hipErrorInvalidValue;                                                        \
    }                                                                                              \
    return hipGetLastError();                                                                      \
  }
  RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
#undef CALL
}

hipError_t launch_flush_gdn(const Args &a, hipStream_t s) {
  const size_t lds = lds_bytes(kKind, a.g.C, 1, a.g.P, a.g.N);
#define CALL(n, r)                                                                                 \
  {                                                                                                \
    switch (a.g.read_copy) {                                                                       \
      case RSSM_READ_NONE: hipLaunchKernelGGL((k_flush<kKind, n, r, RSSM_READ_NONE>), grid_of(a), dim3(kThreads), lds, s, a); break; \
      case RSSM_READ_FP8: hipLaunchKernelGGL((k_flush<kKind, n, r, RSSM_READ_FP8>), grid_of(a), dim3(kThreads), lds, s, a); break; \
      case RSSM_READ_MXFP4: hipLaunchKernelGGL((k_flush<kKind, n, r, RSSM_READ_MXFP4>), grid_of(a), dim3(kThreads), lds, s, a); break; \
      default: return hipErrorInvalidValue;                                                        \
    }                                                                                              \
    return hipGetLastError();                                                                      \
  }
  RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
#undef CALL
}

hipError_t launch_conventional_gdn(const Args &a, hipStream_t s) {
  const size_t lds = lds_bytes(kKind, 1, 1, a.g.P, a.g.N);
#define CALL(n, r)                                                                          \
  {                                                                                         \
    hipLaunchKernelGGL((k_conventional<kKind, n, r>), grid_of(a), dim3(kThreads), lds, s, a); \
    return hipGetLastError();                                                               \
  }
  RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
#undef CALL
}

hipError_t launch_verify_snapshot_gdn(const Args &a, hipStream_t s) {
  const size_t lds = lds_bytes(kKind, a.T, a.T, a.g.P, a.g.N);
#define CALL(n, r)                                                                                  \
  {                                                                                                 \
    hipLaunchKernelGGL((k_verify_snapshot<kKind, n, r>), grid_of(a), dim3(kThreads), lds, s, a);    \
    return hipGetLastError();                                                                       \
  }
  RSSM_DISPATCH(a.g.N, rgw_for(a.g.P), CALL)
#undef CALL
}

}  // namespace rssm
