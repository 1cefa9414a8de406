// Streaming GEMV / small-M launchers of q6sb, q6sb_bf16 (see mv.h).
#include "mv.h"

namespace qg {
QG_MV_INSTANTIATE(6)
QG_MV_INSTANTIATE(16)
}  // namespace qg
