// Streaming GEMV / small-M launchers of q4a32, q3g32 (see mv.h).
#include "mv.h"

namespace qg {
QG_MV_INSTANTIATE(10)
QG_MV_INSTANTIATE(17)
}  // namespace qg
