// Streaming GEMV / small-M launchers of q4g64, q4g128, q4g32h (see mv.h).
#include "mv.h"

namespace qg {
QG_MV_INSTANTIATE(8)
QG_MV_INSTANTIATE(9)
QG_MV_INSTANTIATE(11)
}  // namespace qg
