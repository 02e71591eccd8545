// Kernel instantiations: GruCell, float32 projections.
#include "launch.hpp"

namespace pararnn {
#define PARARNN_NEWTON_CASE_gru_f32(KK, WW) PARARNN_NEWTON_CASE(GruCell, false, KK, WW)
#define PARARNN_ADJOINT_CASE_gru_f32(KK, WW) PARARNN_ADJOINT_CASE(GruCell, false, KK, WW)
PARARNN_DEFINE_LAUNCHERS(gru_f32, GruCell, false, PARARNN_GRU_EXTRA)
PARARNN_DEFINE_SEQ_LAUNCHER(gru_f32, GruCell, false)
}  // namespace pararnn
