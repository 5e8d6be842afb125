// Launchers that record the call instead of launching: the host-side validation layer
// (rssm_api.hip) is exercised under AddressSanitizer / UndefinedBehaviorSanitizer on a machine
// without a GPU.  Every launch that validation lets through increments rssm_stub_launches.
#include "../../attention_decode_mamba_amd/csrc/rssm_internal.hpp"

extern "C" int rssm_stub_launches = 0;

namespace rssm {
static hipError_t record() {
  ++rssm_stub_launches;
  return hipSuccess;
}
hipError_t launch_decode(const Args &, hipStream_t) { return record(); }
hipError_t launch_verify(const Args &, hipStream_t) { return record(); }
hipError_t launch_flush(const Args &, hipStream_t) { return record(); }
hipError_t launch_conventional(const Args &, hipStream_t) { return record(); }
hipError_t launch_init(const Args &, hipStream_t) { return record(); }
hipError_t launch_commit(const Args &, hipStream_t) { return record(); }
hipError_t launch_commit_tree(const Args &, hipStream_t) { return record(); }
hipError_t launch_verify_snapshot(const Args &, hipStream_t) { return record(); }
hipError_t launch_commit_snapshot(const Args &, hipStream_t) { return record(); }
hipError_t launch_clear_err(int32_t *, hipStream_t) { return record(); }
hipError_t launch_stream_copy(const void *, void *, size_t, hipStream_t) { return record(); }
}  // namespace rssm
