// KDA kernel instances whose bf16 records are staged in 16-byte chunks.
#include "kind_launch.hpp"

namespace rssm {
template struct KindLaunch<RSSM_KIND_KDA, kStageBf16>;
}  // namespace rssm
