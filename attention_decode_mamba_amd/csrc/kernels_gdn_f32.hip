// Gated DeltaNet kernel instances whose fp32 records are staged in 16-byte chunks.
#include "kind_launch.hpp"

namespace rssm {
template struct KindLaunch<RSSM_KIND_GDN, kStageF32>;
}  // namespace rssm
