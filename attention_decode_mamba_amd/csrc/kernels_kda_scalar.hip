// KDA kernel instances whose records are staged element by element (rows not 16-byte aligned).
#include "kind_launch.hpp"

namespace rssm {
template struct KindLaunch<RSSM_KIND_KDA, kStageScalar>;
}  // namespace rssm
