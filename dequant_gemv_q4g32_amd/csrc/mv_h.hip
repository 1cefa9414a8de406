// Streaming GEMV / small-M launchers of q5g32 (see mv.h).
#include "mv.h"

namespace qg {
QG_MV_INSTANTIATE(18)
}  // namespace qg
