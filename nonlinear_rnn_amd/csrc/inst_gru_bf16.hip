// Kernel instantiations: GruCell, bfloat16 projections.
#include "launch.hpp"

namespace pararnn {
#define PARARNN_NEWTON_CASE_gru_bf16(KK, WW) PARARNN_NEWTON_CASE(GruCell, true, KK, WW)
#define PARARNN_ADJOINT_CASE_gru_bf16(KK, WW) PARARNN_ADJOINT_CASE(GruCell, true, KK, WW)
PARARNN_DEFINE_LAUNCHERS(gru_bf16, GruCell, true, PARARNN_GRU_EXTRA)
}  // namespace pararnn
