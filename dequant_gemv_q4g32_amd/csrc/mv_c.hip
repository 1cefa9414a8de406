// Streaming GEMV / small-M launchers of q4g32, q4g16 (see mv.h).
#include "mv.h"

namespace qg {
QG_MV_INSTANTIATE(4)
QG_MV_INSTANTIATE(7)
}  // namespace qg
