// Kernel instantiations: LstmCell, float32 projections.
#include "launch.hpp"

namespace pararnn {
#define PARARNN_NEWTON_CASE_lstm_f32(KK, WW) PARARNN_NEWTON_CASE(LstmCell, false, KK, WW)
#define PARARNN_ADJOINT_CASE_lstm_f32(KK, WW) PARARNN_ADJOINT_CASE(LstmCell, false, KK, WW)
PARARNN_DEFINE_LAUNCHERS(lstm_f32, LstmCell, false, PARARNN_NO_EXTRA)
PARARNN_DEFINE_SEQ_LAUNCHER(lstm_f32, LstmCell, false)
}  // namespace pararnn
