// Kernel instantiations: LstmCell, bfloat16 projections.
#include "launch.hpp"

namespace pararnn {
#define PARARNN_NEWTON_CASE_lstm_bf16(KK, WW) PARARNN_NEWTON_CASE(LstmCell, true, KK, WW)
#define PARARNN_ADJOINT_CASE_lstm_bf16(KK, WW) PARARNN_ADJOINT_CASE(LstmCell, true, KK, WW)
PARARNN_DEFINE_LAUNCHERS(lstm_bf16, LstmCell, true, PARARNN_NO_EXTRA)
PARARNN_DEFINE_SEQ_LAUNCHER(lstm_bf16, LstmCell, true)
}  // namespace pararnn
