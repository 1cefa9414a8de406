// Streaming GEMV / small-M launchers of q2sb, q2sb_bf16 (see mv.h).
#include "mv.h"

namespace qg {
QG_MV_INSTANTIATE(2)
QG_MV_INSTANTIATE(12)
}  // namespace qg
