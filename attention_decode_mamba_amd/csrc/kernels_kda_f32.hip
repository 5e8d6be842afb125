// KDA kernel instances whose fp32 records are staged in 16-byte chunks.
#include "kind_launch.hpp"

namespace rssm {
template struct KindLaunch<RSSM_KIND_KDA, kStageF32>;
}  // namespace rssm
