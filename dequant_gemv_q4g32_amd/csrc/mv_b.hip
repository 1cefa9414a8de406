// Streaming GEMV / small-M launchers of q3sb, q3sb_bf16 (see mv.h).
#include "mv.h"

namespace qg {
QG_MV_INSTANTIATE(3)
QG_MV_INSTANTIATE(13)
}  // namespace qg
