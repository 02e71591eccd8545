// Kernel instantiations: GruCell, bfloat16 projections, block-sequential
// time blocks (the long-sequence default with many channels), compiled with
// their own scheduler options (build.py).
#include "launch.hpp"

namespace pararnn {
PARARNN_DEFINE_SEQ_LAUNCHER(gru_bf16, GruCell, true)
}  // namespace pararnn
