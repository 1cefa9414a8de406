// Streaming GEMV / small-M launchers of q5sb, q5sb_bf16 (see mv.h).
#include "mv.h"

namespace qg {
QG_MV_INSTANTIATE(5)
QG_MV_INSTANTIATE(15)
}  // namespace qg
